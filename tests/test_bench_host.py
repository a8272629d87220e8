"""Host logic of bench.py (no GPU): the one-GPU refusal, and the algorithmic
byte count of a step against an item-by-item count on small workloads."""
import json
import os
import subprocess
import sys

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def count_bytes(wl, window, new_tokens):
    """Every byte a step must move, request by request and token by token."""
    c = wl.cfg
    kv, io = bench.ELEM[c.kv_dtype], bench.ELEM[c.io_dtype]
    bs, hkv, hq, d, T = c.block_size, c.n_kv_heads, c.n_q_heads, c.head_dim, new_tokens
    total = 0
    for L in (int(x) for x in wl.context_lens):
        first = max(L - window, 0) if window > 0 else 0
        for t in range(first, L):
            total += 2 * hkv * d * kv          # K and V of token t: read, or written when new
        total += T * hq * d * io * 2           # q read, out written
        total += T * 2 * hkv * d * io          # k_new, v_new read
        total += T * 2 * (d // 2) * 4          # cos and sin rows of each new position
        last = (L - 1) // bs
        total += 4 * (last - first // bs + 1)  # table entries of the blocks read
        total += 4 + 4                         # position and length
    if c.kv_dtype == "fp8":
        total += 4 * hkv * 4                   # K and V scales and their inverses
    return total


@pytest.mark.parametrize("kv", ["bf16", "fp8", "f32"])
@pytest.mark.parametrize("window,new_tokens", [(0, 1), (0, 3), (5, 1), (20, 2), (1000, 1)])
def test_algorithmic_bytes_counts_every_item(kv, window, new_tokens):
    lens = [3, 16, 17, 40, 129]
    io = "f32" if kv == "f32" else "bf16"
    wl = workloads.custom_workload(lens, n_q_heads=8, n_kv_heads=2, head_dim=64, block_size=16,
                                   kv_dtype=kv, io_dtype=io, rope_theta=1.0e4, seed=1)
    assert bench.algorithmic_bytes(wl, window, new_tokens) == count_bytes(wl, window, new_tokens)


def test_traffic_is_reported_only_for_the_kernel_it_was_measured_on(monkeypatch):
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        rec = json.load(fh)
    name = "llama3_8b_b64_gqa4_d128_bf16"
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: rec[name]["kernel_hash"])
    assert bench.measured_traffic(name, 1.0) == rec[name]["bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.measured_traffic(name, 1.0) is None
    assert bench.measured_traffic("no_such_workload", 1.0) is None


@pytest.mark.parametrize("k,tp", [(3, 8), (5, 8), (2, 4)])
def test_tensor_parallel_shard_keeps_the_requests_and_splits_the_heads(k, tp):
    """``--tp``: one GPU's share keeps every request, length and block table
    and holds Hkv/tp KV heads with their Hq/tp query heads (the same group),
    so its algorithmic bytes are the KV and head-proportional terms over tp."""
    full, shard = workloads.make_workload(k), workloads.shard_workload(k, tp)
    assert shard.cfg.n_kv_heads * tp == full.cfg.n_kv_heads
    assert shard.cfg.n_q_heads * tp == full.cfg.n_q_heads
    assert shard.cfg.group == full.cfg.group
    assert (shard.context_lens == full.context_lens).all()
    assert (shard.block_tables == full.block_tables).all()
    assert shard.num_blocks == full.num_blocks and shard.cfg.name.endswith(f"_tp{tp}shard")
    c = full.cfg
    per_batch = int((4 * ((full.context_lens.astype("int64") + c.block_size - 1) // c.block_size) + 8).sum())
    rope = full.batch * c.head_dim * 4
    head_part = bench.algorithmic_bytes(full) - per_batch - rope
    assert bench.algorithmic_bytes(shard) == head_part // tp + per_batch + rope


def test_tensor_parallel_shard_needs_divisible_heads():
    with pytest.raises(ValueError):
        workloads.shard_workload(1, 8)          # 4 KV heads
    with pytest.raises(ValueError):
        workloads.shard_workload(2, 3)


@pytest.mark.parametrize("window,new_tokens", [(0, 1), (5, 1), (0, 3)])
def test_attention_flops_count_every_attended_token(window, new_tokens):
    """The reported arithmetic intensity's FLOPs: 4 D per query head and
    attended token, counted token by token."""
    wl = workloads.custom_workload([1, 7, 40], n_q_heads=8, n_kv_heads=2, head_dim=64,
                                   block_size=16, kv_dtype="bf16", io_dtype="bf16")
    want = 0
    for L in wl.context_lens.tolist():
        for i in range(new_tokens):
            visible = L - new_tokens + i + 1
            want += 4 * 8 * 64 * (min(visible, window) if window else visible)
    assert bench.attention_flops(wl, window, new_tokens) == want
