"""The pool layout helpers (argument marshalling of the binding) against the
byte-offset formulas of the library header, on the CPU."""
import numpy as np
import pytest
import torch

from paged_kv_decode_step_amd import pool_io

import problem


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bs", [16, 32, 64])
def test_pool_io_permutes_follow_the_header_formulas(kv, d, bs):
    nb, hkv = 3, 2
    n_el = nb * hkv * bs * d
    ids = torch.arange(n_el, dtype=torch.int64).reshape(nb, hkv, bs, d)
    kphys = pool_io.k_logical_to_physical(ids, kv).contiguous().reshape(-1).numpy()
    vphys = pool_io.v_logical_to_physical(ids, kv).contiguous().reshape(-1).numpy()
    assert kphys.shape == (n_el,) and vphys.shape == (n_el,)
    assert tuple(pool_io.k_logical_to_physical(ids, kv).shape) == pool_io.k_shape(nb, hkv, bs, d, kv)
    assert tuple(pool_io.v_logical_to_physical(ids, kv).shape) == pool_io.v_shape(nb, hkv, bs, d, kv)
    n, h, t, dd = np.meshgrid(np.arange(nb), np.arange(hkv), np.arange(bs), np.arange(d),
                              indexing="ij")
    kw = dict(hkv=hkv, bs=bs, head_dim=d, kv_dtype=kv)
    ki = problem.k_elem_index(n, h, t, dd, **kw)
    vi = problem.v_elem_index(n, h, t, dd, **kw)
    logical = ids.numpy()
    assert np.array_equal(kphys[ki], logical)
    assert np.array_equal(vphys[vi], logical)
    # and back
    back_k = pool_io.k_physical_to_logical(torch.from_numpy(kphys).reshape(pool_io.k_shape(nb, hkv, bs, d, kv)))
    back_v = pool_io.v_physical_to_logical(torch.from_numpy(vphys).reshape(pool_io.v_shape(nb, hkv, bs, d, kv)))
    assert torch.equal(back_k, ids) and torch.equal(back_v, ids)


def test_one_tile_is_whole_kib_chunks():
    for kv, e in (("f32", 4), ("bf16", 2), ("fp8", 1)):
        for d in (64, 128):
            assert (16 * d * e) % 1024 == 0
