"""Pins of the oracle's decode step: closed forms, invariants, library and
brute-force agreement, and planted mistakes that the pins must catch.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.variants import brute_force_attention, padded_static_batch, split_merge

import problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small(lengths, kv="bf16", io="bf16", hq=8, hkv=2, d=16, bs=4, seed=11, **kw):
    return workloads.custom_workload(lengths, n_q_heads=hq, n_kv_heads=hkv,
                                     head_dim=d, block_size=bs, kv_dtype=kv,
                                     io_dtype=io, seed=seed, **kw)


def run(wl, arrs=None):
    arrs = arrs if arrs is not None else problem.build(wl)
    return arrs, problem.oracle_step(wl, arrs)


# ---------------------------------------------------------------- workloads
def test_config1_lengths_come_from_the_static_batch_figure():
    g = json.load(open(os.path.join(GOLDEN, "static_batch_example.json")))
    lens = [p + n for p, n in zip(g["prompt_tokens"], g["generated_tokens"])]
    assert max(lens) == g["padded_max_length"]
    wl = workloads.make_workload(1)
    assert list(wl.context_lens) == lens
    assert wl.num_blocks == 96


def test_block_tables_waste_bounded_by_last_block():
    g = json.load(open(os.path.join(GOLDEN, "paged_kv_waste_example.json")))
    waste = 1 - g["used_tokens"] / g["reserved_tokens"]
    assert waste >= g["contiguous_waste_fraction_at_least"]
    bs = g["example_block_tokens"]
    blocks = -(-g["used_tokens"] // bs)
    assert blocks * bs - g["used_tokens"] < bs
    for k in (1, 2, 3, 4, 5):
        wl = workloads.make_workload(k)
        nb = wl.n_blocks_used()
        slack = nb * wl.cfg.block_size - wl.context_lens
        assert np.all((slack >= 0) & (slack < wl.cfg.block_size))
        # every used block appears once, tails are -1
        used = np.concatenate([wl.block_tables[b, :n] for b, n in enumerate(nb)])
        assert len(np.unique(used)) == len(used)
        assert used.min() >= 0 and used.max() < wl.num_blocks
        for b, n in enumerate(nb):
            assert np.all(wl.block_tables[b, n:] == -1)


def test_config_recipes():
    w5 = workloads.make_workload(5)
    long = w5.context_lens >= 16384
    assert long.sum() == 51 and w5.batch == 512
    assert np.all((w5.context_lens[~long] >= 64) & (w5.context_lens[~long] <= 512))
    w3 = workloads.make_workload(3)
    assert w3.context_lens.min() >= 16 and w3.context_lens.max() <= 8192
    w4 = workloads.make_workload(4)
    assert w4.context_lens.min() >= 1024 and w4.context_lens.max() <= 32768
    for k in (1, 2, 3, 4, 5):
        wl = workloads.make_workload(k)
        assert np.array_equal(wl.positions, wl.context_lens - 1)


# ---------------------------------------------------------------- append
@pytest.mark.parametrize("kv,io", [("f32", "f32"), ("bf16", "bf16"), ("fp8", "bf16")])
def test_append_touches_only_slot_L_minus_1(kv, io):
    wl = small([1, 4, 5, 9, 16], kv=kv, io=io)
    arrs, res = run(wl)
    bs = wl.cfg.block_size
    changed = np.zeros(wl.num_blocks * wl.cfg.n_kv_heads * bs, bool).reshape(
        wl.num_blocks, wl.cfg.n_kv_heads, bs)
    for b in range(wl.batch):
        L = int(wl.context_lens[b])
        phys = wl.block_tables[b, (L - 1) // bs]
        changed[phys, :, (L - 1) % bs] = True
        assert np.array_equal(res["k_pool"][phys, :, (L - 1) % bs], res["k_app"][b])
        assert np.array_equal(res["v_pool"][phys, :, (L - 1) % bs], res["v_app"][b])
    same_k = (res["k_pool"] == arrs["k_pool"]).all(axis=-1)
    assert np.all(same_k | changed)
    same_v = (res["v_pool"] == arrs["v_pool"]).all(axis=-1)
    assert np.all(same_v | changed)


def test_append_codes_follow_the_pinned_recipe():
    wl = small([3, 7], kv="fp8", io="bf16", d=32)
    arrs, res = run(wl)
    c, s = oracle.rope_rows_f32(wl.cfg.rope_theta, 32, [2])
    k32 = oracle.bf16_bits_to_f32(arrs["k_new"][0])
    y = oracle.rope_k_f32(k32, c[0], s[0])
    inv = oracle.fp8_inverse_scale(arrs["k_scale"])
    want = oracle.fp8_encode(y * inv[:, None])
    assert np.array_equal(res["k_app"][0], want)
    # bf16 value of v_new round-trips through a bf16 cache unchanged
    wl2 = small([3, 7])
    arrs2, res2 = run(wl2)
    assert np.array_equal(res2["v_app"], arrs2["v_new"])


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("kv,io", [("f32", "f32"), ("bf16", "bf16"), ("fp8", "bf16")])
def test_one_token_context_returns_v_exactly(kv, io):
    wl = small([1, 1, 1], kv=kv, io=io)
    arrs, res = run(wl)
    g = wl.cfg.group
    for b in range(wl.batch):
        for hq in range(wl.cfg.n_q_heads):
            v = oracle.kv_to_f64(res["v_app"][b][:, None, :], kv, arrs["v_scale"])[hq // g, 0]
            assert np.array_equal(res["out"][b, hq], v)


def test_identical_keys_give_mean_of_values():
    wl = small([37], kv="f32", io="f32", hq=4, hkv=2)
    arrs = problem.build(wl)
    # every cached key equals the appended key -> all scores equal
    res0 = problem.oracle_step(wl, arrs)
    kp = arrs["k_pool"].copy()
    kp[:] = res0["k_app"][0][None, :, None, :]
    arrs["k_pool"] = kp
    res = problem.oracle_step(wl, arrs)
    kc = oracle.gather_request(res["v_pool"], wl.block_tables[0], 37, wl.cfg.block_size)
    mean = kc.astype(np.float64).mean(axis=1)                  # [Hkv, D]
    for hq in range(4):
        assert np.max(np.abs(res["out"][0, hq] - mean[hq // 2])) < 1e-14


def test_zero_query_gives_mean_of_values():
    wl = small([23, 40], kv="bf16", io="bf16")
    arrs = problem.build(wl)
    arrs["q"] = np.zeros_like(arrs["q"])
    res = problem.oracle_step(wl, arrs)
    for b in range(2):
        L = int(wl.context_lens[b])
        vc = oracle.kv_to_f64(oracle.gather_request(res["v_pool"], wl.block_tables[b], L, 4), "bf16")
        for hq in range(8):
            assert np.max(np.abs(res["out"][b, hq] - vc[hq // 4].mean(0))) < 1e-14


def test_hand_worked_two_token_example():
    # D = 2, theta arbitrary (only frequency is 1), position 1.
    # cached key k0 = (a, b) (already rotated), new key (0, 0) -> rotated (0, 0)
    # q = (x, y) rotated by 1 rad; scores s0 = q_rot . k0 / sqrt 2, s1 = 0.
    wl = small([2], kv="f32", io="f32", hq=1, hkv=1, d=2, bs=2)
    arrs = problem.build(wl)
    a, b_, x, y = 0.75, -1.25, 0.5, 2.0
    v0, v1 = np.array([1.5, -2.0]), np.array([0.25, 4.0])
    phys = wl.block_tables[0, 0]
    arrs["k_pool"][phys, 0, 0] = [a, b_]
    arrs["v_pool"][phys, 0, 0] = v0
    arrs["q"][0, 0] = [x, y]
    arrs["k_new"][0, 0] = [0.0, 0.0]
    arrs["v_new"][0, 0] = v1
    res = problem.oracle_step(wl, arrs)
    qr = (x * math.cos(1) - y * math.sin(1), y * math.cos(1) + x * math.sin(1))
    s0 = (qr[0] * a + qr[1] * b_) / math.sqrt(2)
    w0 = math.exp(s0)
    want = (w0 * v0 + v1) / (w0 + 1)
    assert np.max(np.abs(res["out"][0, 0] - want)) < 1e-15


# ---------------------------------------------------------------- invariants
def test_linear_and_affine_in_values():
    wl = small([13, 30, 5], kv="f32", io="f32")
    arrs = problem.build(wl)
    # values on a 2**-12 grid so that scaling by 4 and shifting by 0.5 are exact
    for key in ("v_pool", "v_new"):
        arrs[key] = (np.round(arrs[key] * 4096) / 4096).astype(np.float32)
    base = problem.oracle_step(wl, arrs)["out"]
    a2 = dict(arrs)
    a2["v_pool"] = arrs["v_pool"] * np.float32(4.0)
    a2["v_new"] = arrs["v_new"] * np.float32(4.0)
    assert np.allclose(problem.oracle_step(wl, a2)["out"], 4.0 * base, rtol=0, atol=1e-13)
    a3 = dict(arrs)
    a3["v_pool"] = arrs["v_pool"] + np.float32(0.5)
    a3["v_new"] = arrs["v_new"] + np.float32(0.5)
    assert np.allclose(problem.oracle_step(wl, a3)["out"], base + 0.5, rtol=0, atol=1e-13)


@pytest.mark.parametrize("kv,io", [("f32", "f32"), ("bf16", "bf16"), ("fp8", "bf16")])
def test_block_permutation_invariance_is_bit_exact(kv, io):
    wl = small([9, 17, 3, 12], kv=kv, io=io)
    arrs = problem.build(wl)
    base = problem.oracle_step(wl, arrs)["out"]
    rng = np.random.default_rng(5)
    perm = rng.permutation(wl.num_blocks)            # new position of block i
    a2 = dict(arrs)
    a2["k_pool"] = np.empty_like(arrs["k_pool"])
    a2["v_pool"] = np.empty_like(arrs["v_pool"])
    a2["k_pool"][perm] = arrs["k_pool"]
    a2["v_pool"][perm] = arrs["v_pool"]
    wl2 = workloads.Workload(wl.cfg, wl.context_lens, wl.positions,
                             np.where(wl.block_tables >= 0, perm[np.maximum(wl.block_tables, 0)], -1).astype(np.int32),
                             wl.num_blocks, wl.seeds)
    assert np.array_equal(problem.oracle_step(wl2, a2)["out"], base)


@pytest.mark.parametrize("kv,io", [("f32", "f32"), ("bf16", "bf16"), ("fp8", "bf16")])
def test_equals_padded_static_batch(kv, io):
    wl = small([1, 17, 64, 5, 33], kv=kv, io=io)
    arrs, res = run(wl)
    dense = padded_static_batch(
        k_pool_after=res["k_pool"], v_pool_after=res["v_pool"], kv_dtype=kv,
        io_dtype=io, q=arrs["q"], positions=wl.positions,
        block_tables=wl.block_tables, context_lens=wl.context_lens,
        block_size=wl.cfg.block_size, rope_theta=wl.cfg.rope_theta,
        k_scale=arrs["k_scale"], v_scale=arrs["v_scale"])
    assert np.max(np.abs(dense - res["out"])) < 1e-13


def test_gqa_equals_mha_with_repeated_kv():
    wl = small([21, 8], kv="bf16", io="bf16", hq=8, hkv=2)
    arrs, res = run(wl)
    g = 4
    wl_mha = workloads.custom_workload([21, 8], n_q_heads=8, n_kv_heads=8, head_dim=16,
                                       block_size=4, kv_dtype="bf16", io_dtype="bf16", seed=11)
    assert np.array_equal(wl_mha.block_tables, wl.block_tables)
    a2 = dict(arrs)
    a2["k_pool"] = np.repeat(arrs["k_pool"], g, axis=1)
    a2["v_pool"] = np.repeat(arrs["v_pool"], g, axis=1)
    a2["k_new"] = np.repeat(arrs["k_new"], g, axis=1)
    a2["v_new"] = np.repeat(arrs["v_new"], g, axis=1)
    res2 = problem.oracle_step(wl_mha, a2)
    assert np.max(np.abs(res2["out"] - res["out"])) < 1e-15


def test_split_merge_equals_unsplit():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((8, 32))
    k = rng.standard_normal((2, 301, 32)) * 3
    v = rng.standard_normal((2, 301, 32))
    whole = oracle.attention_request(q, k, v)
    for chunk in (1, 7, 64, 300, 301, 1000):
        assert np.max(np.abs(split_merge(q, k, v, chunk) - whole)) < 1e-14


# ---------------------------------------------------------------- libraries
def test_matches_torch_sdpa_float64():
    wl = small([40, 1, 77], kv="bf16", io="bf16", hq=8, hkv=2, d=32, bs=8)
    arrs, res = run(wl)
    for b in range(wl.batch):
        L = int(wl.context_lens[b])
        kc = oracle.kv_to_f64(oracle.gather_request(res["k_pool"], wl.block_tables[b], L, 8), "bf16")
        vc = oracle.kv_to_f64(oracle.gather_request(res["v_pool"], wl.block_tables[b], L, 8), "bf16")
        qr = oracle.rope_f64(oracle.io_to_f64(arrs["q"][b], "bf16"), int(wl.positions[b]), wl.cfg.rope_theta)
        kt = torch.from_numpy(np.repeat(kc, 4, axis=0))       # [Hq, L, D]
        vt = torch.from_numpy(np.repeat(vc, 4, axis=0))
        qt = torch.from_numpy(qr)[:, None, :]                   # [Hq, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, 0].numpy()
        assert np.max(np.abs(ref - res["out"][b])) < 1e-12


def test_matches_mpmath_brute_force_tiny():
    wl = small([3, 6], kv="bf16", io="bf16", hq=2, hkv=1, d=4, bs=2)
    arrs, res = run(wl)
    for b in range(wl.batch):
        L = int(wl.context_lens[b])
        kc = oracle.kv_to_f64(oracle.gather_request(res["k_pool"], wl.block_tables[b], L, 2), "bf16")
        vc = oracle.kv_to_f64(oracle.gather_request(res["v_pool"], wl.block_tables[b], L, 2), "bf16")
        q = oracle.io_to_f64(arrs["q"][b], "bf16")
        bf = brute_force_attention(q, kc, vc, int(wl.positions[b]), wl.cfg.rope_theta)
        got = res["out"][b]
        for hq in range(2):
            for j in range(4):
                assert abs(float(bf[hq][j]) - got[hq, j]) < 1e-13


# ---------------------------------------------------------------- planted mistakes
def test_pins_catch_a_planted_mistake_in_the_scale(monkeypatch):
    import oracle.decode as dec

    def wrong(q_rot, k, v):      # forgets 1/sqrt(D)
        hq, d = q_rot.shape
        g = hq // k.shape[0]
        out = np.empty((hq, d))
        for h in range(hq):
            s = k[h // g] @ q_rot[h]
            w = np.exp(s - s.max())
            out[h] = w @ v[h // g] / w.sum()
        return out
    wl = small([40, 9], kv="bf16", io="bf16", hq=8, hkv=2, d=32, bs=8)
    arrs = problem.build(wl)
    good = problem.oracle_step(wl, arrs)["out"]
    monkeypatch.setattr(dec, "attention_request", wrong)
    bad = problem.oracle_step(wl, arrs)["out"]
    # the SDPA pin would see this
    assert np.max(np.abs(bad - good)) > 1e-3


def test_pins_catch_a_planted_head_mapping_mistake():
    # query head hq reading KV head hq % Hkv instead of hq // G breaks GQA == MHA
    wl = small([21, 8], kv="bf16", io="bf16", hq=8, hkv=2)
    arrs, res = run(wl)
    L = 21
    kc = oracle.kv_to_f64(oracle.gather_request(res["k_pool"], wl.block_tables[0], L, 4), "bf16")
    vc = oracle.kv_to_f64(oracle.gather_request(res["v_pool"], wl.block_tables[0], L, 4), "bf16")
    qr = oracle.rope_f64(oracle.io_to_f64(arrs["q"][0], "bf16"), 20, wl.cfg.rope_theta)
    idx = np.arange(8) % 2
    wrong = oracle.attention_request(qr, kc[idx], vc[idx])
    assert np.max(np.abs(wrong - res["out"][0])) > 1e-3


def test_pins_catch_a_planted_rope_sign_mistake():
    # rotating by -angle breaks the relative-position identity used in the pins
    rng = np.random.default_rng(9)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    def wrong(x, p, th):
        return oracle.rope_f64(x, -p, th)
    lhs = wrong(q, 3, 1e4) @ oracle.rope_f64(k, 10, 1e4)
    rhs = q @ oracle.rope_f64(k, 7, 1e4)
    assert abs(lhs - rhs) > 1e-6
