"""Upload a host-built problem to the GPU library, run it, read it back.

Used by the ``gpu`` tests.  Inputs come from ``problem.build`` (the oracle's
codecs) or, for pools too large for the host, from values drawn on the device
and cast with torch; expected values always come from the oracle.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import paged_kv_decode_step_amd as pkv
import workloads
from paged_kv_decode_step_amd import pool_io

DEV = "cuda:0"


def io_to_torch(arr: np.ndarray, io: str) -> torch.Tensor:
    if io == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, np.float32)).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(DEV).view(torch.bfloat16)


def io_from_torch(t: torch.Tensor) -> np.ndarray:
    """Device output -> float64 numpy (exact widening)."""
    return t.float().cpu().numpy().astype(np.float64)


def codes_to_torch(arr: np.ndarray, kv: str) -> torch.Tensor:
    if kv == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, np.float32)).to(DEV)
    if kv == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(arr, np.uint8)).to(DEV)


def codes_from_torch(t: torch.Tensor, kv: str) -> np.ndarray:
    a = t.cpu().numpy()
    if kv == "bf16":
        return a.view(np.uint16)
    return a


def bits(a: np.ndarray) -> np.ndarray:
    """Bit patterns for exact comparison (NaN-safe)."""
    a = np.ascontiguousarray(a)
    return a.view({4: np.uint32, 2: np.uint16, 1: np.uint8}[a.dtype.itemsize])


class Run:
    """A pool plus the device tensors of one step."""

    def __init__(self, wl: workloads.Workload, arrs: dict, *, waves_per_cu: int = 0,
                 min_units: int = None, piece_cost: int = None, young_weight: int = None,
                 odd_weight: int = None,
                 max_position: int = None, tables=None):
        c = wl.cfg
        self.wl, self.arrs = wl, arrs
        self.pool = pkv.KVPool(wl.num_blocks, c.block_size, c.n_kv_heads, c.head_dim,
                               c.kv_dtype)
        self.pool.set_rope(c.rope_theta, max_position or max(wl.max_position, 1))
        if c.kv_dtype == "fp8":
            self.pool.set_fp8_scales(arrs["k_scale"], arrs["v_scale"])
        if (waves_per_cu or min_units or piece_cost is not None or young_weight is not None
                or odd_weight is not None):
            self.pool.set_tuning(waves_per_cu, min_units or 16,
                                 -1 if piece_cost is None else piece_cost,
                                 -1 if young_weight is None else young_weight,
                                 -1 if odd_weight is None else odd_weight)
        pool_io.write_logical(self.pool, codes_to_torch(arrs["k_pool"], c.kv_dtype),
                              codes_to_torch(arrs["v_pool"], c.kv_dtype))
        self.q = io_to_torch(arrs["q"], c.io_dtype)
        self.k_new = io_to_torch(arrs["k_new"], c.io_dtype)
        self.v_new = io_to_torch(arrs["v_new"], c.io_dtype)
        self.positions = torch.from_numpy(wl.positions.astype(np.int32)).to(DEV)
        tb = wl.block_tables if tables is None else tables
        self.tables = torch.from_numpy(np.ascontiguousarray(tb, np.int32)).to(DEV)
        self.lens = torch.from_numpy(wl.context_lens.astype(np.int32)).to(DEV)
        self.out = torch.full_like(self.q, float("nan"))

    def step(self):
        pkv.decode_step(self.pool, self.q, self.k_new, self.v_new, self.positions,
                        self.tables, self.lens, self.out)
        torch.cuda.synchronize()
        return self

    def out_f64(self) -> np.ndarray:
        return io_from_torch(self.out)

    def pools(self):
        k, v = pool_io.read_logical(self.pool)
        kv = self.wl.cfg.kv_dtype
        return codes_from_torch(k, kv), codes_from_torch(v, kv)

    def close(self):
        self.pool.close()


def tolerance(kv: str) -> float:
    """Row-wise relative tolerance of the output (max |err| / max |ref| per
    (request, query head) row): 1e-2 for a bf16 cache, 5e-2 for fp8 (against
    the oracle on dequantised values); the fp32 path computes in fp32
    throughout, so 1e-4 is asserted for it."""
    return {"bf16": 1e-2, "fp8": 5e-2, "f32": 1e-4}[kv]


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return num / np.maximum(den, 1e-300)


# ---- pools drawn on the device (full-size workloads) -------------------------
def device_pool_codes(wl: workloads.Workload, chunk_blocks: int = 4096):
    """Draw the cached K/V on the device (float32 N(0,1)) and cast them to the
    cache type with torch: bf16 by RNE, fp8 by per-head amax/448 scales with
    saturation.  Yields (first_block, k_codes, v_codes) logical chunks; for
    fp8 also returns the scales (computed over the whole pool first)."""
    c = wl.cfg
    nb = wl.num_blocks
    scales = None
    if c.kv_dtype == "fp8":
        amax_k = torch.zeros(c.n_kv_heads, device=DEV)
        amax_v = torch.zeros(c.n_kv_heads, device=DEV)
        for b0 in range(0, nb, chunk_blocks):
            n = min(chunk_blocks, nb - b0)
            k = workloads.device_normals(wl, "k_cache", DEV, b0, n)
            amax_k = torch.maximum(amax_k, k.abs().amax(dim=(0, 2, 3)))
            del k
            v = workloads.device_normals(wl, "v_cache", DEV, b0, n)
            amax_v = torch.maximum(amax_v, v.abs().amax(dim=(0, 2, 3)))
            del v
        k_scale = (amax_k / 448.0).float().cpu().numpy()
        v_scale = (amax_v / 448.0).float().cpu().numpy()
        scales = (k_scale, v_scale)

    def cast(x, which):
        if c.kv_dtype == "bf16":
            return x.to(torch.bfloat16).view(torch.int16)
        if c.kv_dtype == "f32":
            return x
        s = scales[0] if which == "k" else scales[1]
        inv = torch.from_numpy(oracle.fp8_inverse_scale(s)).to(DEV)
        y = (x * inv.view(1, -1, 1, 1)).clamp(-448.0, 448.0)
        return y.to(torch.float8_e4m3fn).view(torch.uint8)

    def chunks():
        for b0 in range(0, nb, chunk_blocks):
            n = min(chunk_blocks, nb - b0)
            k = cast(workloads.device_normals(wl, "k_cache", DEV, b0, n), "k")
            v = cast(workloads.device_normals(wl, "v_cache", DEV, b0, n), "v")
            yield b0, k, v

    return chunks, scales


def host_io_arrays(wl: workloads.Workload) -> dict:
    c = wl.cfg
    enc = (lambda x: x) if c.io_dtype == "f32" else oracle.bf16_bits_from_f32
    return {"q": enc(workloads.host_normals(wl, "q")),
            "k_new": enc(workloads.host_normals(wl, "k_new")),
            "v_new": enc(workloads.host_normals(wl, "v_new"))}


def mini_problem(wl: workloads.Workload, b: int, k_blocks: np.ndarray, v_blocks: np.ndarray,
                 io: dict, scales) -> tuple:
    """Request b alone, its blocks renumbered 0..n-1: inputs for the oracle."""
    c = wl.cfg
    n = k_blocks.shape[0]
    mini_wl = workloads.Workload(
        c, wl.context_lens[b:b + 1], wl.positions[b:b + 1],
        np.arange(n, dtype=np.int32)[None, :], n, wl.seeds)
    arrs = {"k_pool": k_blocks, "v_pool": v_blocks,
            "q": io["q"][b:b + 1], "k_new": io["k_new"][b:b + 1],
            "v_new": io["v_new"][b:b + 1],
            "k_scale": None if scales is None else scales[0],
            "v_scale": None if scales is None else scales[1]}
    return mini_wl, arrs
