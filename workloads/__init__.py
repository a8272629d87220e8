"""Seeded synthetic decode-step workloads.

This module is shared by the tests, the benchmark and the oracle's tests.  It
draws only the *inputs* of a paged decode step: context lengths, the physical
block assignment (block tables), positions and raw float32 N(0, 1) values for
the cached K/V, the new query and the new K/V.  It holds none of the method's
arithmetic: no rounding to a storage type, no RoPE, no attention.  Whoever
consumes the raw float32 values casts them to the storage dtype it needs.

Workload shapes follow the pages' own workloads:

* the tiny ragged batch takes its lengths from the padded static-batch figure
  of "TensorRT-LLM Guide: High-Throughput GPU Inference Engine" (section "The
  Problem: The Memory-Bandwidth Wall and Static Batching Inefficiencies"):
  prompts of 128, 512 and 64 tokens with 10, 500 and 20 generated tokens give
  contexts of 138, 1012 and 84;
* a fixed-size block pool with per-request block tables is the paged KV cache
  of "Scaling TensorRT-LLM: Kernel Fusion and Inflight Batching in
  Production" (section "The Paged KV-Cache: vLLM Borrowed by TensorRT-LLM");
* the heterogeneous batch mixes short chat turns with a long-context tail as in
  that page's "The Two-Engine Trick for Chat Workloads".

Conventions: ``context_lens[b]`` counts the new token, so after the step the
request holds ``L_b`` tokens and the new token lands in slot ``L_b - 1``;
``positions[b] = L_b - 1``.  Block tables are int32 ``[B, max_blocks]``,
row-major, with ``-1`` in the entries past ``ceil(L_b / block_size)``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence

import numpy as np

__all__ = [
    "Config", "CONFIGS", "Workload", "make_workload", "custom_workload",
    "shard_workload", "host_normals", "device_normals",
]


@dataclasses.dataclass(frozen=True)
class Config:
    """Shape and length recipe of one synthetic workload."""

    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    kv_dtype: str            # "f32", "bf16" or "fp8"
    io_dtype: str            # "f32" or "bf16"
    rope_theta: float
    lengths: str             # recipe tag, see _draw_lengths
    seed: int
    fixed_lengths: Optional[Sequence[int]] = None
    fixed_pool_blocks: Optional[int] = None

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


CONFIGS: Dict[int, Config] = {
    1: Config("tiny_ragged_b3_h4_d64_f32", 3, 4, 4, 64, 16, "f32", "f32",
              1.0e4, "fixed", 1001, fixed_lengths=(138, 1012, 84),
              fixed_pool_blocks=96),
    2: Config("llama3_8b_b64_gqa4_d128_bf16", 64, 32, 8, 128, 16, "bf16",
              "bf16", 5.0e5, "uniform_64_2048", 1002),
    3: Config("llama70b_b256_gqa8_d128_bf16", 256, 64, 8, 128, 16, "bf16",
              "bf16", 5.0e5, "lognormal_1024_clip_16_8192", 1003),
    4: Config("fp8kv_b128_gqa4_d128_bs32", 128, 32, 8, 128, 32, "fp8",
              "bf16", 5.0e5, "uniform_1024_32768", 1004),
    5: Config("hetero_b512_gqa8_d128_bs32", 512, 64, 8, 128, 32, "bf16",
              "bf16", 5.0e5, "bimodal_512", 1005),
}


def _children(seed: int):
    """Fixed-order child streams: lengths, long indices, block permutation,
    K cache, V cache, q/k_new/v_new."""
    ss = np.random.SeedSequence(seed)
    return ss.spawn(6)


def _draw_lengths(cfg: Config, ch) -> np.ndarray:
    rng_len = np.random.default_rng(ch[0])
    tag, b = cfg.lengths, cfg.batch
    if tag == "fixed":
        return np.asarray(cfg.fixed_lengths, dtype=np.int64)
    if tag == "uniform_64_2048":
        return rng_len.integers(64, 2048, size=b, endpoint=True)
    if tag == "uniform_1024_32768":
        return rng_len.integers(1024, 32768, size=b, endpoint=True)
    if tag == "lognormal_1024_clip_16_8192":
        x = rng_len.lognormal(mean=math.log(1024.0), sigma=1.0, size=b)
        return np.clip(np.rint(x), 16, 8192).astype(np.int64)
    if tag == "bimodal_512":
        n_long = int(round(0.1 * b))
        rng_idx = np.random.default_rng(ch[1])
        long_idx = rng_idx.choice(b, size=n_long, replace=False)
        lens = rng_len.integers(64, 512, size=b, endpoint=True)
        lens[long_idx] = rng_len.integers(16384, 131072, size=n_long,
                                          endpoint=True)
        return lens
    raise ValueError(f"unknown length recipe {tag!r}")


@dataclasses.dataclass
class Workload:
    """Everything about a decode step except the cached and new values."""

    cfg: Config
    context_lens: np.ndarray        # int32 [B]
    positions: np.ndarray           # int32 [B]
    block_tables: np.ndarray        # int32 [B, max_blocks], -1 tails
    num_blocks: int
    seeds: Sequence[np.random.SeedSequence]

    @property
    def batch(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_position(self) -> int:
        return int(self.positions.max()) + 1 if self.batch else 1

    def n_blocks_used(self) -> np.ndarray:
        bs = self.cfg.block_size
        return (self.context_lens.astype(np.int64) + bs - 1) // bs


def _assign_blocks(lens: np.ndarray, bs: int, num_blocks: int, rng,
                   max_blocks: Optional[int] = None):
    """Hand out a seeded permutation of all pool blocks in request order."""
    need = (lens.astype(np.int64) + bs - 1) // bs
    total = int(need.sum())
    if total > num_blocks:
        raise ValueError("pool too small for the requested lengths")
    perm = rng.permutation(num_blocks).astype(np.int32)
    mb = int(need.max()) if max_blocks is None else int(max_blocks)
    mb = max(mb, 1)
    tables = np.full((lens.shape[0], mb), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        tables[b, :n] = perm[off:off + n]
        off += int(n)
    return tables


def make_workload(cfg_or_index, batch: Optional[int] = None) -> Workload:
    """Lengths and block tables of one of the five configurations.

    ``batch`` keeps only the first ``batch`` requests (same draw), for scaled
    down parity cases; the pool is then sized for the kept requests.
    """
    cfg = CONFIGS[cfg_or_index] if isinstance(cfg_or_index, int) else cfg_or_index
    ch = _children(cfg.seed)
    lens = _draw_lengths(cfg, ch)
    if batch is not None:
        lens = lens[:batch]
    bs = cfg.block_size
    need = int(((lens + bs - 1) // bs).sum())
    if cfg.fixed_pool_blocks is not None and batch is None:
        num_blocks = cfg.fixed_pool_blocks
    else:
        num_blocks = int(math.ceil(1.05 * need))
    tables = _assign_blocks(lens, bs, num_blocks,
                            np.random.default_rng(ch[2]))
    lens32 = lens.astype(np.int32)
    return Workload(cfg, lens32, (lens32 - 1).astype(np.int32), tables,
                    num_blocks, ch)


def shard_workload(cfg_or_index, tp: int) -> Workload:
    """One GPU's share of a workload when its attention heads are split over
    ``tp`` GPUs: tensor parallelism, which runs a 70B model over 8 GPUs
    ("Lesson 13.17 TensorRT-LLM: NVIDIA's Optimized Inference Engine", section
    "Speculative decoding and running one model across many GPUs") by
    splitting the attention projections across them ("TensorRT-LLM Guide:
    High-Throughput GPU Inference Engine", section "1. Scaling Across NVLink
    with Tensor Parallelism (TP)").  The same requests, lengths and block
    tables, with ``Hkv / tp`` KV heads and their ``Hq / tp`` query heads; the
    shard's cache and new values are drawn from the same streams at the
    shard's shape."""
    cfg = CONFIGS[cfg_or_index] if isinstance(cfg_or_index, int) else cfg_or_index
    if tp < 1 or cfg.n_kv_heads % tp or cfg.n_q_heads % tp:
        raise ValueError(f"{cfg.name}: {cfg.n_q_heads}/{cfg.n_kv_heads} heads do not split over {tp}")
    full = make_workload(cfg)
    shard = dataclasses.replace(cfg, name=f"{cfg.name}_tp{tp}shard", n_q_heads=cfg.n_q_heads // tp,
                                n_kv_heads=cfg.n_kv_heads // tp)
    return Workload(shard, full.context_lens, full.positions, full.block_tables,
                    full.num_blocks, full.seeds)


def custom_workload(lengths: Sequence[int], *, n_q_heads: int, n_kv_heads: int,
                    head_dim: int, block_size: int, kv_dtype: str,
                    io_dtype: str, rope_theta: float = 1.0e4, seed: int = 7,
                    extra_blocks: int = 3, max_blocks: Optional[int] = None,
                    positions: Optional[Sequence[int]] = None) -> Workload:
    """A hand-shaped workload for edge cases (same generation rules)."""
    lens = np.asarray(lengths, dtype=np.int64)
    cfg = Config(f"custom_{seed}", int(lens.shape[0]), n_q_heads, n_kv_heads,
                 head_dim, block_size, kv_dtype, io_dtype, rope_theta,
                 "fixed", seed, fixed_lengths=tuple(int(x) for x in lens))
    ch = _children(seed)
    bs = block_size
    need = int(((lens + bs - 1) // bs).sum())
    num_blocks = need + extra_blocks
    tables = _assign_blocks(lens, bs, num_blocks, np.random.default_rng(ch[2]),
                            max_blocks=max_blocks)
    lens32 = lens.astype(np.int32)
    pos = (lens32 - 1) if positions is None else np.asarray(positions, np.int32)
    return Workload(cfg, lens32, pos.astype(np.int32), tables, num_blocks, ch)


def host_normals(wl: Workload, what: str) -> np.ndarray:
    """Raw float32 N(0, 1) values on the host.

    ``what``: "k_cache" / "v_cache" -> logical ``[num_blocks, Hkv, bs, D]``;
    "q" -> ``[B, Hq, D]``; "k_new" / "v_new" -> ``[B, Hkv, D]``.
    """
    c = wl.cfg
    if what in ("k_cache", "v_cache"):
        rng = np.random.default_rng(wl.seeds[3 if what == "k_cache" else 4])
        shape = (wl.num_blocks, c.n_kv_heads, c.block_size, c.head_dim)
        return rng.standard_normal(shape, dtype=np.float32)
    rng = np.random.default_rng(wl.seeds[5])
    q = rng.standard_normal((wl.batch, c.n_q_heads, c.head_dim), dtype=np.float32)
    k = rng.standard_normal((wl.batch, c.n_kv_heads, c.head_dim), dtype=np.float32)
    v = rng.standard_normal((wl.batch, c.n_kv_heads, c.head_dim), dtype=np.float32)
    return {"q": q, "k_new": k, "v_new": v}[what]


def device_normals(wl: Workload, what: str, device, block_start: int = 0,
                   n_blocks: Optional[int] = None):
    """Raw float32 N(0, 1) values drawn on a torch device.

    For pools too large to draw on the host.  Cache values are drawn per
    chunk of blocks, each chunk from its own generator seeded by the
    workload's stream and the chunk's first block, so any chunking of the
    same range reproduces the same values only when the same chunk bounds are
    used; callers use ``chunk_blocks`` multiples from block 0.
    """
    import torch

    c = wl.cfg
    which = {"k_cache": 3, "v_cache": 4}[what]
    if n_blocks is None:
        n_blocks = wl.num_blocks - block_start
    seed = int(wl.seeds[which].generate_state(1, dtype=np.uint64)[0] % (2**63))
    g = torch.Generator(device=device)
    g.manual_seed((seed + 1000003 * block_start) % (2**63))
    shape = (n_blocks, c.n_kv_heads, c.block_size, c.head_dim)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)
