"""Move storage codes between the logical cache layout and the pool.

The logical layout is ``[blocks, Hkv, block_size, D]``; the pool's physical
layout is the one ``include/pkv.h`` documents (K in 16-byte rows
``[blocks, Hkv, D/x, block_size, x]``, V as ``[blocks, Hkv, D, block_size]``).
These are permutes of stored codes (float32, bf16 bits as int16, E4M3 codes
as uint8) for filling and inspecting a pool; nothing here is arithmetic.
"""
from __future__ import annotations

import torch

_ELEM = {"f32": 4, "bf16": 2, "fp8": 1}
_TORCH = {"f32": torch.float32, "bf16": torch.int16, "fp8": torch.uint8}


def storage_dtype(kv_dtype: str):
    return _TORCH[kv_dtype]


def k_logical_to_physical(k: torch.Tensor, kv_dtype: str) -> torch.Tensor:
    n, h, bs, d = k.shape
    x = 16 // _ELEM[kv_dtype]
    return k.reshape(n, h, bs, d // x, x).permute(0, 1, 3, 2, 4)


def k_physical_to_logical(k: torch.Tensor) -> torch.Tensor:
    n, h, dx, bs, x = k.shape
    return k.permute(0, 1, 3, 2, 4).reshape(n, h, bs, dx * x)


def v_logical_to_physical(v: torch.Tensor) -> torch.Tensor:
    return v.permute(0, 1, 3, 2)


def v_physical_to_logical(v: torch.Tensor) -> torch.Tensor:
    return v.permute(0, 1, 3, 2)


def write_logical(pool, k_codes: torch.Tensor, v_codes: torch.Tensor, first_block: int = 0):
    """Copy logical-layout codes for blocks [first_block, first_block + n)."""
    n = k_codes.shape[0]
    ks, vs = pool.k_storage(), pool.v_storage()
    ks[first_block:first_block + n].copy_(k_logical_to_physical(k_codes, pool.kv_dtype))
    vs[first_block:first_block + n].copy_(v_logical_to_physical(v_codes))


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
