"""Python binding of ``libpkv.so``, the paged-KV decode step for MI355X.

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI declared in ``include/pkv.h``.  PyTorch supplies
device memory and the stream.  There is no fallback: if the library is not
built, or no GPU is present, the calls raise.

Names follow the C ABI: ``KVPool`` wraps ``kv_pool_*`` and ``decode_step``
calls ``decode_step``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch  # noqa: F401  (binds libpkv to torch's HIP runtime, loaded first)

__all__ = [
    "KVPool", "decode_step", "PkvError", "load_library", "LIB_PATH", "DTYPES",
    "check_decode_args", "rope_table_host", "plan_host", "tile_tokens",
    "EXPORTED_SYMBOLS", "HOST_SYMBOLS", "BlockAllocator", "decode_step_multi", "stream_read",
    "decode_step_noalloc", "TIMELINE_LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")
# the same library with per-wavefront phase stamps (kv_pool_read_timeline)
TIMELINE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv_timeline.so")

DTYPES = {"f32": 0, "bf16": 1, "fp8": 2}
_ELEM = {"f32": 4, "bf16": 2, "fp8": 1}
_STATUS = {0: "OK", -1: "INVALID", -2: "UNSUPPORTED", -3: "OOM", -4: "HIP",
           -5: "STATE", -6: "DEVICE_DATA"}

# every function include/pkv.h declares
EXPORTED_SYMBOLS = (
    "kv_pool_create", "kv_pool_destroy", "kv_pool_set_rope",
    "kv_pool_set_fp8_scales", "kv_pool_get_info", "kv_pool_layout",
    "kv_pool_rope_table", "decode_step",
    "kv_pool_device_errors", "kv_pool_set_tuning", "kv_pool_enable_timing",
    "kv_pool_read_timing", "pkv_last_error",
    "pkv_check_decode_args", "pkv_rope_table_host", "pkv_plan_host",
    "pkv_tile_tokens", "kv_pool_copy_blocks", "kv_pool_set_window", "decode_step_multi",
    "pkv_alloc_create", "pkv_alloc_destroy", "pkv_alloc_stats", "pkv_alloc_refcount",
    "pkv_seq_add", "pkv_seq_fork", "pkv_seq_release", "pkv_seq_info",
    "pkv_alloc_prepare_step", "pkv_stream_read", "decode_step_noalloc",
    "kv_pool_read_timeline",
)


class PkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class _Info(ctypes.Structure):
    _fields_ = [
        ("num_blocks", ctypes.c_int64), ("block_size", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32), ("kv_elem_bytes", ctypes.c_int32),
        ("tile_bytes", ctypes.c_int32), ("k_base", ctypes.c_void_p),
        ("v_base", ctypes.c_void_p), ("k_bytes", ctypes.c_int64),
        ("v_bytes", ctypes.c_int64), ("rope_cos", ctypes.c_void_p),
        ("rope_sin", ctypes.c_void_p), ("rope_max_position", ctypes.c_int32),
        ("rope_theta", ctypes.c_double), ("has_fp8_scales", ctypes.c_int32),
        ("device", ctypes.c_int32), ("n_waves", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_int64), ("ring_tiles", ctypes.c_int32),
        ("min_units", ctypes.c_int32), ("piece_cost", ctypes.c_int32),
        ("young_weight_pct", ctypes.c_int32), ("n_first", ctypes.c_int32),
        ("odd_weight_pct", ctypes.c_int32), ("window", ctypes.c_int32),
    ]


# the entry points that need no GPU: argument checks, the RoPE table, the
# work-partition replay and the block allocator (a host-only build of the
# library exports just these)
HOST_SYMBOLS = (
    "pkv_last_error", "pkv_check_decode_args", "pkv_rope_table_host", "pkv_plan_host",
    "pkv_tile_tokens", "pkv_alloc_create", "pkv_alloc_destroy", "pkv_alloc_stats",
    "pkv_alloc_refcount", "pkv_seq_add", "pkv_seq_fork", "pkv_seq_release", "pkv_seq_info",
    "pkv_alloc_prepare_step",
)

_lib = None


def load_library(path: str = LIB_PATH, host_only: bool = False):
    """Load libpkv.so once and declare its signatures.  ``host_only`` loads
    a build of the host-only entry points alone (``HOST_SYMBOLS``), such as
    the sanitizer-instrumented one the CPU tests use."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise PkvError(-5, f"{path} is not built; run paged_kv_decode_step_amd.build")
    lib = ctypes.CDLL(path)
    P, I32, I64, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    IP = ctypes.POINTER(ctypes.c_int32)
    FP = ctypes.POINTER(ctypes.c_float)
    sig = {
        "kv_pool_create": (I32, [I64, I32, I32, I32, I32, ctypes.POINTER(P)]),
        "kv_pool_destroy": (I32, [P]),
        "kv_pool_set_rope": (I32, [P, D, I32]),
        "kv_pool_set_fp8_scales": (I32, [P, FP, FP]),
        "kv_pool_get_info": (I32, [P, ctypes.POINTER(_Info)]),
        "kv_pool_layout": (I32, [P, ctypes.POINTER(P), ctypes.POINTER(P),
                                 ctypes.POINTER(I64), IP]),
        "kv_pool_rope_table": (I32, [P, ctypes.POINTER(P), ctypes.POINTER(P), IP]),
        "decode_step": (I32, [P, P, P, P, I32, P, P, I32, P, I32, I32, P, P]),
        "decode_step_noalloc": (I32, [P, P, P, P, I32, P, P, I32, P, I32, I32, P, P]),
        "kv_pool_device_errors": (I32, [P, ctypes.POINTER(ctypes.c_uint32)]),
        "kv_pool_set_tuning": (I32, [P, I32, I32, I32, I32, I32]),
        "kv_pool_enable_timing": (I32, [P, I32]),
        "kv_pool_read_timing": (I32, [P, ctypes.POINTER(D), ctypes.POINTER(D),
                                      ctypes.POINTER(I32)]),
        "pkv_last_error": (ctypes.c_char_p, []),
        "pkv_check_decode_args": (I32, [I64, I32, I32, I32, I32, I32, P, P, P, P, P,
                                        I32, P, I32, I32, P]),
        "pkv_rope_table_host": (I32, [D, I32, I32, FP, FP]),
        "pkv_plan_host": (I32, [IP, I32, I32, I32, I32, I32, I32, I32, I32, I32, I32, I32, I32, I32, IP, IP, IP]),
        "pkv_tile_tokens": (I32, []),
        "kv_pool_copy_blocks": (I32, [P, P, I32, P]),
        "kv_pool_set_window": (I32, [P, I32]),
        "decode_step_multi": (I32, [P, P, P, P, I32, I32, P, P, I32, P, I32, I32, P, P]),
        "pkv_alloc_create": (I32, [I64, I32, I32, ctypes.POINTER(P)]),
        "pkv_alloc_destroy": (I32, [P]),
        "pkv_alloc_stats": (I32, [P, ctypes.POINTER(I64), IP]),
        "pkv_alloc_refcount": (I32, [P, I32, IP]),
        "pkv_seq_add": (I32, [P, I32, IP]),
        "pkv_seq_fork": (I32, [P, I32, IP]),
        "pkv_seq_release": (I32, [P, I32]),
        "pkv_seq_info": (I32, [P, I32, IP, IP, IP, I32]),
        "pkv_alloc_prepare_step": (I32, [P, IP, I32, I32, IP, IP, IP, IP, I32, IP]),
        "pkv_stream_read": (I32, [P, I64, P, P]),
        "kv_pool_read_timeline": (I32, [P, P, I32, IP]),
    }
    for name, (res, args) in sig.items():
        if host_only and name not in HOST_SYMBOLS:
            continue
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        raise PkvError(status, _lib.pkv_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


class _CudaArray:
    """A device buffer described for torch.as_tensor (zero copy)."""

    def __init__(self, ptr: int, shape, typestr: str):
        self.__cuda_array_interface__ = {
            "shape": tuple(int(s) for s in shape), "typestr": typestr,
            "data": (int(ptr), False), "version": 2, "strides": None,
        }


class KVPool:
    """Owner of a pool of KV blocks on the current device (``kv_pool_*``)."""

    def __init__(self, num_blocks: int, block_size: int, n_kv_heads: int,
                 head_dim: int, kv_dtype: str):
        lib = load_library()
        self.kv_dtype = kv_dtype
        h = ctypes.c_void_p()
        _check(lib.kv_pool_create(int(num_blocks), int(block_size), int(n_kv_heads),
                                  int(head_dim), DTYPES[kv_dtype], ctypes.byref(h)))
        self._h = h
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        self.n_kv_heads, self.head_dim = int(n_kv_heads), int(head_dim)
        self.device = int(self.info()["device"])      # HIP ordinal the pool lives on

    @property
    def handle(self):
        if self._h is None:
            raise PkvError(-5, "pool is closed")
        return self._h

    def set_rope(self, theta: float, max_position: int) -> None:
        _check(_lib.kv_pool_set_rope(self.handle, float(theta), int(max_position)))

    def set_fp8_scales(self, k_scale: Sequence[float], v_scale: Sequence[float]) -> None:
        n = self.n_kv_heads
        ks = (ctypes.c_float * n)(*[float(x) for x in k_scale])
        vs = (ctypes.c_float * n)(*[float(x) for x in v_scale])
        _check(_lib.kv_pool_set_fp8_scales(self.handle, ks, vs))

    def set_tuning(self, waves_per_cu: int = 0, min_units: int = 16, piece_cost: int = -1,
                   young_weight_pct: int = -1, odd_weight_pct: int = -1) -> None:
        _check(_lib.kv_pool_set_tuning(self.handle, int(waves_per_cu), int(min_units),
                                       int(piece_cost), int(young_weight_pct),
                                       int(odd_weight_pct)))

    def set_window(self, window: int) -> None:
        """Attend to the last ``window`` tokens of each request (0 = all)."""
        _check(_lib.kv_pool_set_window(self.handle, int(window)))

    def copy_blocks(self, pairs, stream=None) -> None:
        """Copy whole blocks, ``pairs`` an int32 ``[n, 2]`` device tensor of
        (source, destination) ids (``kv_pool_copy_blocks``; asynchronous)."""
        if (pairs.dtype != torch.int32 or not pairs.is_contiguous() or pairs.device.type != "cuda"
                or pairs.device.index != self.device):
            raise PkvError(-1, f"pairs must be a contiguous int32 tensor on cuda:{self.device}")
        if pairs.dim() != 2 or pairs.shape[1] != 2:
            raise PkvError(-1, "pairs must be [n, 2]")
        if stream is None:
            stream = torch.cuda.current_stream(pairs.device).cuda_stream
        elif not isinstance(stream, int):
            stream = stream.cuda_stream
        _check(_lib.kv_pool_copy_blocks(self.handle, _ptr(pairs), int(pairs.shape[0]),
                                        ctypes.c_void_p(stream)))

    def enable_timing(self, enable: bool = True) -> None:
        _check(_lib.kv_pool_enable_timing(self.handle, 1 if enable else 0))

    def read_timing(self):
        """(attention ms, merge ms, calls) summed since the last read."""
        a, m, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int32()
        _check(_lib.kv_pool_read_timing(self.handle, ctypes.byref(a), ctypes.byref(m),
                                        ctypes.byref(n)))
        return a.value, m.value, n.value

    def read_timeline(self):
        """``kv_pool_read_timeline``: the last step's per-wavefront records as
        a uint64 array [n_waves, 8] (timeline builds only)."""
        import numpy as np
        cap = int(self.info()["n_waves"])
        rec = np.zeros((cap, 8), dtype=np.uint64)
        n = ctypes.c_int32()
        _check(_lib.kv_pool_read_timeline(self.handle, ctypes.c_void_p(rec.ctypes.data), cap,
                                          ctypes.byref(n)))
        return rec[:min(cap, n.value)]

    def info(self) -> dict:
        inf = _Info()
        _check(_lib.kv_pool_get_info(self.handle, ctypes.byref(inf)))
        return {k: getattr(inf, k) for k, _ in _Info._fields_}

    def layout(self) -> dict:
        """``kv_pool_layout``: K and V base addresses, the byte strides per
        block, KV head and 16-token tile, and the tile's size in bytes."""
        k, v = ctypes.c_void_p(), ctypes.c_void_p()
        st = (ctypes.c_int64 * 3)()
        tb = ctypes.c_int32()
        _check(_lib.kv_pool_layout(self.handle, ctypes.byref(k), ctypes.byref(v), st,
                                   ctypes.byref(tb)))
        return {"k_base": k.value, "v_base": v.value, "byte_strides": tuple(st),
                "tile_bytes": tb.value}

    def rope_table(self):
        """``kv_pool_rope_table``: the device tables as float32 tensors
        ``[max_position, head_dim / 2]`` (cos, sin), zero copy."""
        c, s = ctypes.c_void_p(), ctypes.c_void_p()
        n = ctypes.c_int32()
        _check(_lib.kv_pool_rope_table(self.handle, ctypes.byref(c), ctypes.byref(s),
                                       ctypes.byref(n)))
        shape = (n.value, self.head_dim // 2)
        dev = f"cuda:{self.device}"
        return (torch.as_tensor(_CudaArray(c.value, shape, "<f4"), device=dev),
                torch.as_tensor(_CudaArray(s.value, shape, "<f4"), device=dev))

    def device_errors(self) -> int:
        f = ctypes.c_uint32()
        _check(_lib.kv_pool_device_errors(self.handle, ctypes.byref(f)))
        return int(f.value)

    def _view(self, which: str):
        from . import pool_io

        inf = self.info()
        ptr = inf["k_base"] if which == "k" else inf["v_base"]
        args = (self.num_blocks, self.n_kv_heads, self.block_size, self.head_dim, self.kv_dtype)
        shape = pool_io.k_shape(*args) if which == "k" else pool_io.v_shape(*args)
        typestr = {4: "<f4", 2: "<i2", 1: "|u1"}[_ELEM[self.kv_dtype]]
        return torch.as_tensor(_CudaArray(ptr, shape, typestr), device=f"cuda:{inf['device']}")

    def k_storage(self):
        """Raw K storage as a torch tensor view ``[nb, Hkv, bs/16, D/x, 16, x]``
        (float32 / int16 holding bf16 bits / uint8 E4M3 codes)."""
        return self._view("k")

    def v_storage(self):
        """Raw V storage as a torch tensor view ``[nb, Hkv, bs/16, D/(16g), 4, 16, g, 4]``."""
        return self._view("v")

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            _lib.kv_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _step_args(pool: KVPool, q, k_new, v_new, positions, block_tables, context_lens, out,
               stream):
    """Checked C arguments of ``decode_step`` and ``decode_step_noalloc``."""
    io = {torch.float32: "f32", torch.bfloat16: "bf16"}.get(q.dtype)
    if io is None:
        raise PkvError(-1, f"unsupported io dtype {q.dtype}")
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("out", out),
                    ("positions", positions), ("block_tables", block_tables),
                    ("context_lens", context_lens)):
        if not t.is_contiguous():
            raise PkvError(-1, f"{name} must be contiguous")
        if t.device.type != "cuda" or t.device.index != pool.device:
            raise PkvError(-1, f"{name} must be on the pool's GPU (cuda:{pool.device})")
    for name, t in (("positions", positions), ("block_tables", block_tables),
                    ("context_lens", context_lens)):
        if t.dtype != torch.int32:
            raise PkvError(-1, f"{name} must be int32")
    for name, t in (("k_new", k_new), ("v_new", v_new), ("out", out)):
        if t.dtype != q.dtype:
            raise PkvError(-1, f"{name} must have q's dtype")
    batch = int(q.shape[0])
    hq = int(q.shape[1]) if q.dim() == 3 else 0
    if q.dim() != 3 or q.shape[2] != pool.head_dim or out.shape != q.shape:
        raise PkvError(-1, "q/out must be [B, Hq, head_dim]")
    if tuple(k_new.shape) != (batch, pool.n_kv_heads, pool.head_dim) or k_new.shape != v_new.shape:
        raise PkvError(-1, "k_new/v_new must be [B, Hkv, head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != batch:
        raise PkvError(-1, "block_tables must be [B, max_blocks]")
    if positions.numel() != batch or context_lens.numel() != batch:
        raise PkvError(-1, "positions/context_lens must be [B]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    return (pool.handle, _ptr(q), _ptr(k_new), _ptr(v_new), DTYPES[io], _ptr(positions),
            _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), batch, hq,
            _ptr(out), ctypes.c_void_p(stream))


def decode_step(pool: KVPool, q, k_new, v_new, positions, block_tables,
                context_lens, out, stream=None) -> None:
    """Launch one decode step (asynchronous on ``stream``; torch tensors).

    ``q``/``out`` ``[B, Hq, D]``, ``k_new``/``v_new`` ``[B, Hkv, D]`` in the
    I/O dtype (float32 or bfloat16), ``positions``/``context_lens`` int32
    ``[B]``, ``block_tables`` int32 ``[B, max_blocks]``, all contiguous on the
    pool's device.
    """
    lib = load_library()
    _check(lib.decode_step(*_step_args(pool, q, k_new, v_new, positions, block_tables,
                                       context_lens, out, stream)))


def decode_step_noalloc(pool: KVPool, q, k_new, v_new, positions, block_tables,
                        context_lens, out, stream=None) -> None:
    """``decode_step`` with the split-K workspace in the library's fixed
    per-device array instead of the pool's (``decode_step_noalloc``): nothing
    is allocated; calls that overlap on one GPU race."""
    lib = load_library()
    _check(lib.decode_step_noalloc(*_step_args(pool, q, k_new, v_new, positions, block_tables,
                                               context_lens, out, stream)))


class BlockAllocator:
    """Host block allocator of a paged pool (``pkv_alloc_*`` / ``pkv_seq_*``):
    sequences hold block lists, shared blocks are reference counted, and
    ``prepare_step`` returns a step's block tables, lengths, positions and
    the copy-on-write pairs as numpy arrays."""

    def __init__(self, num_blocks: int, block_size: int, max_seqs: int):
        lib = load_library()
        h = ctypes.c_void_p()
        _check(lib.pkv_alloc_create(int(num_blocks), int(block_size), int(max_seqs),
                                    ctypes.byref(h)))
        self._h = h
        self.num_blocks, self.block_size, self.max_seqs = int(num_blocks), int(block_size), int(max_seqs)

    @property
    def handle(self):
        if self._h is None:
            raise PkvError(-5, "allocator is closed")
        return self._h

    def close(self) -> None:
        if self._h is not None:
            _lib.pkv_alloc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def stats(self):
        """(free blocks, live sequences)."""
        fb, ls = ctypes.c_int64(), ctypes.c_int32()
        _check(_lib.pkv_alloc_stats(self.handle, ctypes.byref(fb), ctypes.byref(ls)))
        return fb.value, ls.value

    def refcount(self, block: int) -> int:
        c = ctypes.c_int32()
        _check(_lib.pkv_alloc_refcount(self.handle, int(block), ctypes.byref(c)))
        return c.value

    def add(self, length: int) -> int:
        s = ctypes.c_int32()
        _check(_lib.pkv_seq_add(self.handle, int(length), ctypes.byref(s)))
        return s.value

    def fork(self, parent: int) -> int:
        s = ctypes.c_int32()
        _check(_lib.pkv_seq_fork(self.handle, int(parent), ctypes.byref(s)))
        return s.value

    def release(self, seq: int) -> None:
        _check(_lib.pkv_seq_release(self.handle, int(seq)))

    def info(self, seq: int):
        """(length, block ids as a list)."""
        import numpy as np

        length, nb = ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.pkv_seq_info(self.handle, int(seq), ctypes.byref(length), ctypes.byref(nb),
                                 None, 0))
        blocks = np.zeros(max(nb.value, 1), dtype=np.int32)
        ip = ctypes.POINTER(ctypes.c_int32)
        _check(_lib.pkv_seq_info(self.handle, int(seq), None, None, blocks.ctypes.data_as(ip),
                                 nb.value))
        return length.value, [int(b) for b in blocks[:nb.value]]

    def prepare_step(self, seq_ids, max_blocks_per_seq: int, max_copies: int = None,
                     out=None):
        """Grow each sequence by one token: (block_tables [B, max_blocks_per_seq],
        context_lens [B], positions [B], copies [n, 2]), int32 numpy arrays.

        ``out``: optional (tables, lens, pos, copies) C-contiguous int32 arrays
        of at least [B, max_blocks_per_seq], [B], [B] and [max_copies, 2] to
        fill instead of new ones (a serving loop reuses them every step); the
        results are views of them."""
        import numpy as np

        ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        b = int(ids.shape[0])
        mc = b if max_copies is None else int(max_copies)
        maxb = int(max_blocks_per_seq)
        if out is None:
            tables = np.empty((max(b, 1), maxb), dtype=np.int32)
            lens = np.empty(max(b, 1), dtype=np.int32)
            pos = np.empty(max(b, 1), dtype=np.int32)
            copies = np.empty((max(mc, 1), 2), dtype=np.int32)
        else:
            tables, lens, pos, copies = out
            for name, a, ndim in (("tables", tables, 2), ("lens", lens, 1), ("pos", pos, 1),
                                  ("copies", copies, 2)):
                if (not isinstance(a, np.ndarray) or a.dtype != np.int32 or a.ndim != ndim
                        or not a.flags["C_CONTIGUOUS"]):
                    raise PkvError(-1, f"out {name} must be a C-contiguous int32 array of {ndim} dims")
            if (tables.shape[0] < b or tables.shape[1] != maxb or lens.shape[0] < b
                    or pos.shape[0] < b or copies.shape[0] < mc or copies.shape[1] != 2):
                raise PkvError(-1, "out arrays are too small for this step")
        n = ctypes.c_int32()
        ip = ctypes.POINTER(ctypes.c_int32)
        _check(_lib.pkv_alloc_prepare_step(self.handle, ids.ctypes.data_as(ip), b,
                                           maxb, tables.ctypes.data_as(ip),
                                           lens.ctypes.data_as(ip), pos.ctypes.data_as(ip),
                                           copies.ctypes.data_as(ip), mc, ctypes.byref(n)))
        return tables[:b], lens[:b], pos[:b], copies[:n.value]


def decode_step_multi(pool: KVPool, q, k_new, v_new, positions, block_tables,
                      context_lens, out, stream=None) -> None:
    """Launch a step with T new tokens per request (``decode_step_multi``):
    ``q``/``out`` ``[B, T, Hq, D]``, ``k_new``/``v_new`` ``[B, T, Hkv, D]``,
    ``positions`` the first new token's position, ``context_lens`` counting
    all T new tokens; query i attends to the tokens ``[0, L - T + i]``."""
    lib = load_library()
    io = {torch.float32: "f32", torch.bfloat16: "bf16"}.get(q.dtype)
    if io is None:
        raise PkvError(-1, f"unsupported io dtype {q.dtype}")
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("out", out),
                    ("positions", positions), ("block_tables", block_tables),
                    ("context_lens", context_lens)):
        if not t.is_contiguous() or t.device.type != "cuda" or t.device.index != pool.device:
            raise PkvError(-1, f"{name} must be contiguous on the pool's GPU (cuda:{pool.device})")
    for name, t in (("positions", positions), ("block_tables", block_tables),
                    ("context_lens", context_lens)):
        if t.dtype != torch.int32:
            raise PkvError(-1, f"{name} must be int32")
    for name, t in (("k_new", k_new), ("v_new", v_new), ("out", out)):
        if t.dtype != q.dtype:
            raise PkvError(-1, f"{name} must have q's dtype")
    if q.dim() != 4 or q.shape[3] != pool.head_dim or out.shape != q.shape:
        raise PkvError(-1, "q/out must be [B, T, Hq, head_dim]")
    batch, tq, hq = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
    if tuple(k_new.shape) != (batch, tq, pool.n_kv_heads, pool.head_dim) or k_new.shape != v_new.shape:
        raise PkvError(-1, "k_new/v_new must be [B, T, Hkv, head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != batch:
        raise PkvError(-1, "block_tables must be [B, max_blocks]")
    if positions.numel() != batch or context_lens.numel() != batch:
        raise PkvError(-1, "positions/context_lens must be [B]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    _check(lib.decode_step_multi(pool.handle, _ptr(q), _ptr(k_new), _ptr(v_new), DTYPES[io], tq,
                                 _ptr(positions), _ptr(block_tables), int(block_tables.shape[1]),
                                 _ptr(context_lens), batch, hq, _ptr(out),
                                 ctypes.c_void_p(stream)))


def stream_read(src, sink, stream=None) -> None:
    """``pkv_stream_read``: read all of the contiguous device tensor ``src``
    once with 16-byte nontemporal loads (asynchronous; the achievable-peak
    reference of the benchmark).  ``sink``: a device tensor of >= 1 KiB."""
    lib = load_library()
    if not src.is_contiguous() or src.device.type != "cuda" or sink.device != src.device:
        raise PkvError(-1, "src and sink must be contiguous tensors on one GPU")
    if sink.numel() * sink.element_size() < 1024:
        raise PkvError(-1, "sink must hold at least 1 KiB")
    if stream is None:
        stream = torch.cuda.current_stream(src.device).cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    nbytes = src.numel() * src.element_size()
    with torch.cuda.device(src.device):
        _check(lib.pkv_stream_read(_ptr(src), int(nbytes), _ptr(sink), ctypes.c_void_p(stream)))


# ---- host-only helpers -----------------------------------------------------
def tile_tokens() -> int:
    return int(load_library().pkv_tile_tokens())


def check_decode_args(*, num_blocks, block_size, n_kv_heads, head_dim, kv_dtype,
                      io_dtype, q=1, k_new=1, v_new=1, positions=1, block_tables=1,
                      max_blocks_per_seq=1, context_lens=1, batch=1, n_q_heads=1,
                      out=1) -> int:
    """Run the library's host-side argument check; returns the status code.
    Pointer arguments are plain integers (no memory is touched)."""
    lib = load_library()
    io = DTYPES.get(io_dtype, io_dtype) if isinstance(io_dtype, str) else io_dtype
    kv = DTYPES.get(kv_dtype, kv_dtype) if isinstance(kv_dtype, str) else kv_dtype
    return int(lib.pkv_check_decode_args(
        int(num_blocks), int(block_size), int(n_kv_heads), int(head_dim), kv, io,
        q, k_new, v_new, positions, block_tables, int(max_blocks_per_seq),
        context_lens, int(batch), int(n_q_heads), out))


def last_error() -> str:
    return load_library().pkv_last_error().decode()


def rope_table_host(theta: float, head_dim: int, max_position: int):
    """The library's RoPE table (numpy float32 ``[max_position, D/2]`` x2)."""
    import numpy as np

    lib = load_library()
    n = max_position * (head_dim // 2)
    c = np.empty(n, dtype=np.float32)
    s = np.empty(n, dtype=np.float32)
    fp = ctypes.POINTER(ctypes.c_float)
    _check(lib.pkv_rope_table_host(float(theta), int(head_dim), int(max_position),
                                   c.ctypes.data_as(fp), s.ctypes.data_as(fp)))
    return c.reshape(max_position, head_dim // 2), s.reshape(max_position, head_dim // 2)


def plan_host(context_lens, n_kv_heads: int, max_tokens: int, n_waves: int,
              min_units: int, piece_cost: int = 0, n_first: int = 0, weight_first: int = 1,
              weight_rest: int = 1, weight_min_share: int = 0, max_pieces: int = 1 << 20,
              weight_odd: int = 100, window: int = 0):
    """Host replay of the kernel's work partition (numpy arrays): pieces
    ``[n, 6]`` and the per-wave split-sequence rows ``[n_waves, 4]``.  The
    first ``n_first`` wavefronts weigh ``weight_first``, the rest
    ``weight_rest``, when there are at least ``weight_min_share`` units per
    wavefront (else those age weights are even); wavefronts of odd
    workgroups (index // 4 odd) are further weighted ``weight_odd`` percent."""
    import numpy as np

    lib = load_library()
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    pieces = np.zeros((max_pieces, 6), dtype=np.int32)
    splits = np.zeros((n_waves, 4), dtype=np.int32)
    n = ctypes.c_int32()
    ip = ctypes.POINTER(ctypes.c_int32)
    _check(lib.pkv_plan_host(lens.ctypes.data_as(ip), int(lens.shape[0]), int(n_kv_heads),
                             int(max_tokens), int(n_waves), int(min_units), int(piece_cost),
                             int(n_first), int(weight_first), int(weight_rest), int(weight_odd),
                             int(weight_min_share), int(window), int(max_pieces),
                             pieces.ctypes.data_as(ip), ctypes.byref(n),
                             splits.ctypes.data_as(ip)))
    return pieces[:min(n.value, max_pieces)], splits
