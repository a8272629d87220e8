"""The C ABI called from plain C, with no Python or torch in the process.

``c_abi_driver.c`` (compiled here with gcc against ``include/pkv.h`` and
``libpkv.so``) grows three requests' contexts from empty to 40 tokens, one
``decode_step`` per token, on inputs from a 32-bit linear congruential
generator, and writes the last step's output and both pools to a file.  The
test draws the same inputs and checks the file:

* bit-equal to the same 40 steps run through the Python binding (the two
  callers marshal the same arguments, so the library cannot tell them apart);
* against the oracle run over the same 40 steps: the pools bit-equal (every
  appended K row is the bf16 rounding of the rotated key, every V row the
  value's code) and the output within the bf16 tolerance.

The CPU test checks that the header compiles as strict C11 and that the
driver links against every entry point it names.
"""
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "paged_kv_decode_step_amd")
SRC = os.path.join(HERE, "c_abi_driver.c")

B, HKV, HQ, D, BS, MAXB, STEPS = 3, 8, 32, 128, 16, 3, 40
THETA, SEED = 5.0e5, 20241203


def compile_driver(out: str) -> None:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-D__HIP_PLATFORM_AMD__", "-isystem", "/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           SRC, "-o", out, "-L" + PKG, "-lpkv", "-Wl,-rpath," + PKG,
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, " ".join(cmd) + "\n" + res.stdout + res.stderr


def test_driver_compiles_and_links_as_c(tmp_path):
    if not os.path.exists(os.path.join(PKG, "libpkv.so")):
        pytest.skip("libpkv.so not built")
    compile_driver(str(tmp_path / "c_abi_driver"))


def draw_inputs():
    """Per step (q, k_new, v_new) as bf16 bit patterns, drawn as the driver
    draws them: LCG x <- 1664525 x + 1013904223 (mod 2^32); a value is
    (x >> 8) / 2^23 - 1 in float32 (exact), truncated to its top 16 bits."""
    n = B * HQ * D + 2 * B * HKV * D
    raw = np.empty(STEPS * n, dtype=np.uint32)
    x = SEED
    for i in range(raw.size):
        x = (x * 1664525 + 1013904223) & 0xFFFFFFFF
        raw[i] = x
    f = (raw >> 8).astype(np.float32) * np.float32(1.0 / 8388608.0) - np.float32(1.0)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16).reshape(STEPS, n)
    nq, nk = B * HQ * D, B * HKV * D
    return [(s[:nq].reshape(B, HQ, D), s[nq:nq + nk].reshape(B, HKV, D),
             s[nq + nk:].reshape(B, HKV, D)) for s in bits]


def tables():
    return np.arange(B * MAXB, dtype=np.int32).reshape(B, MAXB)


@pytest.mark.gpu
def test_c_driver_matches_binding_and_oracle(tmp_path):
    import torch

    import oracle
    import paged_kv_decode_step_amd as pkv
    from paged_kv_decode_step_amd import pool_io

    import gpu_problem as gp

    exe = str(tmp_path / "c_abi_driver")
    compile_driver(exe)
    dump = str(tmp_path / "c_abi_out.bin")
    print(f"c abi driver: {B} requests x {STEPS} steps", flush=True)
    res = subprocess.run([exe, dump], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    raw = np.fromfile(dump, dtype=np.uint8)

    nb = B * MAXB
    out_bytes = B * HQ * D * 2
    pool_bytes = nb * HKV * BS * D * 2
    assert raw.size == out_bytes + 2 * pool_bytes
    c_out = raw[:out_bytes].view(np.uint16).reshape(B, HQ, D)
    kshape = pool_io.k_shape(nb, HKV, BS, D, "bf16")
    vshape = pool_io.v_shape(nb, HKV, BS, D, "bf16")
    c_k = pool_io.k_physical_to_logical(
        torch.from_numpy(raw[out_bytes:out_bytes + pool_bytes].view(np.int16).reshape(kshape)))
    c_v = pool_io.v_physical_to_logical(
        torch.from_numpy(raw[out_bytes + pool_bytes:].view(np.int16).reshape(vshape)))
    c_k = c_k.contiguous().numpy().view(np.uint16)
    c_v = c_v.contiguous().numpy().view(np.uint16)

    steps = draw_inputs()
    tab = tables()

    # the same steps through the Python binding
    pool = pkv.KVPool(nb, BS, HKV, D, "bf16")
    try:
        pool.set_rope(THETA, STEPS)
        pool.k_storage().zero_()
        pool.v_storage().zero_()
        dt = torch.from_numpy(tab).to(gp.DEV)
        out = torch.empty(B, HQ, D, dtype=torch.bfloat16, device=gp.DEV)
        for s, (q, kn, vn) in enumerate(steps):
            pos = torch.full((B,), s, dtype=torch.int32, device=gp.DEV)
            lens = torch.full((B,), s + 1, dtype=torch.int32, device=gp.DEV)
            pkv.decode_step(pool, gp.io_to_torch(q, "bf16"), gp.io_to_torch(kn, "bf16"),
                            gp.io_to_torch(vn, "bf16"), pos, dt, lens, out)
        torch.cuda.synchronize()
        assert pool.device_errors() == 0
        py_out = out.view(torch.int16).cpu().numpy().view(np.uint16)
        py_k, py_v = (gp.codes_from_torch(t, "bf16") for t in pool_io.read_logical(pool))
    finally:
        pool.close()
    assert np.array_equal(c_out, py_out), "output differs from the Python caller's"
    assert np.array_equal(c_k, py_k) and np.array_equal(c_v, py_v), "pools differ"

    # the oracle over the same steps
    kp = np.zeros((nb, HKV, BS, D), np.uint16)
    vp = np.zeros((nb, HKV, BS, D), np.uint16)
    for s, (q, kn, vn) in enumerate(steps):
        ref = oracle.decode_step(
            k_pool=kp, v_pool=vp, kv_dtype="bf16", io_dtype="bf16", q=q, k_new=kn, v_new=vn,
            positions=np.full(B, s, np.int32), block_tables=tab,
            context_lens=np.full(B, s + 1, np.int32), block_size=BS, rope_theta=THETA)
        kp, vp = ref["k_pool"], ref["v_pool"]
    assert np.array_equal(c_k, kp), "K pool differs from the oracle's"
    assert np.array_equal(c_v, vp), "V pool differs from the oracle's"
    err = gp.row_rel_err(oracle.bf16_bits_to_f64(c_out), ref["out"])
    assert err.max() <= gp.tolerance("bf16"), err.max()
