"""Move storage codes between the logical cache layout and the pool.

The logical layout is ``[blocks, Hkv, block_size, D]``; the pool's physical
layout is the one ``include/pkv.h`` documents.  A block is ``block_size / 16``
tiles of 16 tokens, and each (block, head, tile) holds its K and its V as
whole 1 KiB chunks in the order the matrix-core operands are read:

* K tile ``[D/x][16 tokens][x]`` with ``x = 16 / element_size``;
* V tile ``[D/(16 g)][4][16][g][4]`` with ``g = 4 / element_size``: for chunk
  ``c``, lane ``16 lq + lr`` holds tokens ``4 lq .. 4 lq + 3`` of the dims
  ``16 (g c + k) + lr``, ``k < g``.

These are permutes of stored codes (float32, bf16 bits as int16, E4M3 codes
as uint8) for filling and inspecting a pool; nothing here is arithmetic.
They work on torch tensors on any device.
"""
from __future__ import annotations

import torch

_ELEM = {"f32": 4, "bf16": 2, "fp8": 1}
_TORCH = {"f32": torch.float32, "bf16": torch.int16, "fp8": torch.uint8}
TILE = 16


def storage_dtype(kv_dtype: str):
    return _TORCH[kv_dtype]


def k_shape(nb: int, hkv: int, bs: int, d: int, kv_dtype: str):
    x = 16 // _ELEM[kv_dtype]
    return (nb, hkv, bs // TILE, d // x, TILE, x)


def v_shape(nb: int, hkv: int, bs: int, d: int, kv_dtype: str):
    g = 4 // _ELEM[kv_dtype]
    return (nb, hkv, bs // TILE, d // (16 * g), 4, 16, g, 4)


def k_logical_to_physical(k: torch.Tensor, kv_dtype: str) -> torch.Tensor:
    n, h, bs, d = k.shape
    x = 16 // _ELEM[kv_dtype]
    return k.reshape(n, h, bs // TILE, TILE, d // x, x).permute(0, 1, 2, 4, 3, 5)


def k_physical_to_logical(k: torch.Tensor) -> torch.Tensor:
    n, h, tpb, dx, t, x = k.shape
    return k.permute(0, 1, 2, 4, 3, 5).reshape(n, h, tpb * t, dx * x)


def v_logical_to_physical(v: torch.Tensor, kv_dtype: str) -> torch.Tensor:
    n, h, bs, d = v.shape
    g = 4 // _ELEM[kv_dtype]
    # [n, h, tile, lq, e, c, k, lr] -> [n, h, tile, c, lq, lr, k, e]
    return v.reshape(n, h, bs // TILE, 4, 4, d // (16 * g), g, 16).permute(0, 1, 2, 5, 3, 7, 6, 4)


def v_physical_to_logical(v: torch.Tensor) -> torch.Tensor:
    n, h, tpb, c, lq, lr, g, e = v.shape
    # [n, h, tile, c, lq, lr, k, e] -> [n, h, tile, lq, e, c, k, lr]
    return v.permute(0, 1, 2, 4, 7, 3, 6, 5).reshape(n, h, tpb * lq * e, c * g * lr)


def write_logical(pool, k_codes: torch.Tensor, v_codes: torch.Tensor, first_block: int = 0):
    """Copy logical-layout codes for blocks [first_block, first_block + n)."""
    n = k_codes.shape[0]
    ks, vs = pool.k_storage(), pool.v_storage()
    ks[first_block:first_block + n].copy_(k_logical_to_physical(k_codes, pool.kv_dtype))
    vs[first_block:first_block + n].copy_(v_logical_to_physical(v_codes, pool.kv_dtype))


def read_logical(pool, first_block: int = 0, n: int = None):
    """Logical-layout copies of the codes of blocks [first_block, first_block + n)."""
    ks, vs = pool.k_storage(), pool.v_storage()
    if n is None:
        n = ks.shape[0] - first_block
    k = k_physical_to_logical(ks[first_block:first_block + n]).contiguous()
    v = v_physical_to_logical(vs[first_block:first_block + n]).contiguous()
    return k, v


def gather_blocks_logical(pool, block_ids: torch.Tensor):
    """Logical-layout copies of the given blocks (any order)."""
    ks, vs = pool.k_storage(), pool.v_storage()
    k = k_physical_to_logical(ks.index_select(0, block_ids)).contiguous()
    v = v_physical_to_logical(vs.index_select(0, block_ids)).contiguous()
    return k, v
