"""Build ``libpkv.so`` (HIP kernels + C ABI) in-tree for gfx950.

Usage: ``python -m paged_kv_decode_step_amd.build [--timeline]`` (or
``build()``).  The library lands next to this file, where the binding loads
it from.  The sources compile to objects in parallel (the attention kernels
once per cache type), which are then linked.  ``--timeline`` builds
``libpkv_timeline.so`` instead: the same kernels with per-wavefront phase
stamps (``kv_pool_read_timeline``), for measurement only.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpkv.so")
OBJ_DIR = os.path.join(HERE, "_build")
TIMELINE_LIB = os.path.join(HERE, "libpkv_timeline.so")
TIMELINE_OBJ_DIR = os.path.join(HERE, "_build_timeline")
DECODE = os.path.join(CSRC, "decode.hip")
KV_KINDS = (0, 1, 2)            # KV_F32, KV_BF16, KV_FP8: one object each
OTHER_SOURCES = ["blocks.hip", "stream_read.hip", "noalloc.hip", "dispatch.cpp", "pkv_host.cpp",
                 "host_api.cpp", "block_alloc.cpp"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # the appended key's RoPE is specified as separate fp32 multiplies and
    # adds; nothing may be contracted into an FMA unless written so
    "-ffp-contract=off",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_jobs(decode_src: str = DECODE, obj_dir: str = OBJ_DIR, defines=()) -> list:
    """(command, object) pairs: decode.hip once per cache type, then the rest."""
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC, *defines]
    jobs = []
    for kv in KV_KINDS:
        obj = os.path.join(obj_dir, f"decode_kv{kv}.o")
        jobs.append(([hipcc(), *FLAGS, *inc, f"-DPKV_KV={kv}", "-c", decode_src, "-o", obj], obj))
    for src in OTHER_SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        jobs.append(([hipcc(), *FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    return jobs


def build(verbose: bool = False, decode_src: str = DECODE, out: str = LIB,
          obj_dir: str = OBJ_DIR, timeline: bool = False) -> str:
    """Compile every source (in parallel) and link the shared library
    (with ``timeline``, the timeline build at its own path)."""
    if timeline and out == LIB:
        out, obj_dir = TIMELINE_LIB, TIMELINE_OBJ_DIR
    os.makedirs(obj_dir, exist_ok=True)
    jobs = compile_jobs(decode_src, obj_dir, ["-DPKV_TIMELINE"] if timeline else [])

    def run(cmd):
        return subprocess.run(cmd, capture_output=True, text=True)

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        results = list(ex.map(run, [cmd for cmd, _ in jobs]))
    for (cmd, _), res in zip(jobs, results):
        if res.returncode != 0:
            sys.stderr.write(" ".join(cmd) + "\n" + res.stdout + res.stderr)
            raise RuntimeError("hipcc failed building libpkv.so")
        if verbose:
            sys.stderr.write(res.stderr)
    tmp = out + ".tmp"
    res = run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC",
               *[obj for _, obj in jobs], "-o", tmp])
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("linking libpkv.so failed")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, timeline="--timeline" in sys.argv[1:]))
