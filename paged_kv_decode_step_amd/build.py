"""Build ``libpkv.so`` (HIP kernels + C ABI) in-tree for gfx950.

Usage: ``python -m paged_kv_decode_step_amd.build`` (or ``build()``).  The
library lands next to this file, where the binding loads it from.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpkv.so")
SOURCES = [os.path.join(HERE, "csrc", "decode.hip"),
           os.path.join(HERE, "csrc", "blocks.hip"),
           os.path.join(HERE, "csrc", "stream_read.hip"),
           os.path.join(HERE, "csrc", "noalloc.hip"),
           os.path.join(HERE, "csrc", "pkv_host.cpp"),
           os.path.join(HERE, "csrc", "block_alloc.cpp")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def command(out: str = LIB) -> list:
    return [
        hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        # the appended key's RoPE is specified as separate fp32 multiplies
        # and adds; nothing may be contracted into an FMA unless written so
        "-ffp-contract=off",
        # packed fp32 VALU ops are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        *SOURCES, "-o", out,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libpkv.so")
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
