"""Test-side construction of a decode-step problem on the host.

Draws the seeded raw values of a workload and encodes them into cache and
I/O storage with the oracle's codecs.  Also restates, from the library
header's byte-offset formulas, where each element of the oracle's logical
cache layout ``[num_blocks, Hkv, bs, D]`` lives in the library's pool.
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads

NAN_CODE = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0),
            "fp8": np.uint8(0x7F)}
STORAGE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}
ELEM = {"f32": 4, "bf16": 2, "fp8": 1}


def encode_io(x32: np.ndarray, io_dtype: str) -> np.ndarray:
    if io_dtype == "f32":
        return np.asarray(x32, np.float32)
    return oracle.bf16_bits_from_f32(x32)


def build(wl: workloads.Workload, poison: bool = False) -> dict:
    """Host arrays of one step: logical pools (codes), inputs, scales."""
    c = wl.cfg
    kraw = workloads.host_normals(wl, "k_cache")
    vraw = workloads.host_normals(wl, "v_cache")
    k_scale = v_scale = None
    if c.kv_dtype == "fp8":
        k_scale = (np.abs(kraw).max(axis=(0, 2, 3)) / np.float32(448.0)).astype(np.float32)
        v_scale = (np.abs(vraw).max(axis=(0, 2, 3)) / np.float32(448.0)).astype(np.float32)
        inv_k = oracle.fp8_inverse_scale(k_scale)
        inv_v = oracle.fp8_inverse_scale(v_scale)
        kp = oracle.fp8_encode(kraw * inv_k[None, :, None, None])
        vp = oracle.fp8_encode(vraw * inv_v[None, :, None, None])
    elif c.kv_dtype == "bf16":
        kp = oracle.bf16_bits_from_f32(kraw)
        vp = oracle.bf16_bits_from_f32(vraw)
    else:
        kp, vp = kraw, vraw
    if poison:
        poison_unused(wl, kp, vp)
    q = encode_io(workloads.host_normals(wl, "q"), c.io_dtype)
    kn = encode_io(workloads.host_normals(wl, "k_new"), c.io_dtype)
    vn = encode_io(workloads.host_normals(wl, "v_new"), c.io_dtype)
    return dict(k_pool=kp, v_pool=vp, q=q, k_new=kn, v_new=vn,
                k_scale=k_scale, v_scale=v_scale)


def poison_unused(wl, kp, vp):
    """NaN in every slot no request reads before the step: slot L-1 of each
    request, the tail of each last block and every unassigned block."""
    c = wl.cfg
    bs = c.block_size
    nan = NAN_CODE[c.kv_dtype]
    used = np.zeros(wl.num_blocks, dtype=bool)
    for b in range(wl.batch):
        L = int(wl.context_lens[b])
        nb = (L + bs - 1) // bs
        used[wl.block_tables[b, :nb]] = True
        last = int(wl.block_tables[b, (L - 1) // bs])
        kp[last, :, (L - 1) % bs:, :] = nan
        vp[last, :, (L - 1) % bs:, :] = nan
    kp[~used] = nan
    vp[~used] = nan


def oracle_step(wl, arrs) -> dict:
    c = wl.cfg
    return oracle.decode_step(
        k_pool=arrs["k_pool"], v_pool=arrs["v_pool"], kv_dtype=c.kv_dtype,
        io_dtype=c.io_dtype, q=arrs["q"], k_new=arrs["k_new"],
        v_new=arrs["v_new"], positions=wl.positions,
        block_tables=wl.block_tables, context_lens=wl.context_lens,
        block_size=c.block_size, rope_theta=c.rope_theta,
        k_scale=arrs["k_scale"], v_scale=arrs["v_scale"])


# ---- physical layout of the library, restated from include/pkv.h ----------
def k_elem_index(n, h, t, d, *, hkv, bs, head_dim, kv_dtype):
    """Element index in the K pool of (block n, head h, token t, dim d),
    from the byte-offset formula of the library header."""
    e = ELEM[kv_dtype]
    x = 16 // e
    tpb = bs // 16
    tile_bytes = 16 * head_dim * e
    base = ((n * hkv + h) * tpb + t // 16) * tile_bytes
    off = ((d // x) * 16 + t % 16) * 16 + (d % x) * e
    return (base + off) // e


def v_elem_index(n, h, t, d, *, hkv, bs, head_dim, kv_dtype):
    """Element index in the V pool of (block n, head h, token t, dim d)."""
    e = ELEM[kv_dtype]
    g = 4 // e
    tpb = bs // 16
    tile_bytes = 16 * head_dim * e
    base = ((n * hkv + h) * tpb + t // 16) * tile_bytes
    nt = d // 16
    c, k = nt // g, nt % g
    t16 = t % 16
    off = (c * 64 + (t16 // 4) * 16 + d % 16) * 16 + (4 * k + t16 % 4) * e
    return (base + off) // e


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per output row ``(b, hq)``: ``max_d |got - ref| / max_d |ref|``."""
    num = np.abs(got.astype(np.float64) - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return num / np.maximum(den, 1e-300)
