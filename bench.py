#!/usr/bin/env python3
"""Benchmark of one paged-KV decode step on one MI355X.

A step is one ``decode_step`` call (RoPE, append, paged attention over the
whole ragged batch, split merge) for one layer of the workload.  Inputs are
synthetic, drawn on the device, and resident in HBM before timing starts.
Consecutive steps cycle over enough independent pools ("layers") that each
step reads a cold working set of at least 1 GB, larger than the 256 MB
Infinity Cache.

Prints one JSON line: the metric is the algorithmic HBM bandwidth of the
step (bytes the method must move / step time) with its fraction of the
8 TB/s peak and the decode tokens/s per layer; ``roofline`` reports the
attention kernel's own duration from HIP events on its launch stream;
``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "paged decode attention: HBM GB/s (% of peak) and decode tokens/s per layer"
ELEM = {"f32": 4, "bf16": 2, "fp8": 1}


def algorithmic_bytes(wl, window: int = 0, new_tokens: int = 1) -> int:
    """Bytes the step must move: cached K/V read once per KV head, the new
    K/V written, q/k_new/v_new read, out written, the block-table entries,
    positions and lengths, the RoPE rows and (fp8) the scales.  With an
    attention window of W tokens only the last W tokens of a request (the
    new one included) and the table entries of their blocks count."""
    c = wl.cfg
    s_kv, s_io = ELEM[c.kv_dtype], ELEM[c.io_dtype]
    L = wl.context_lens.astype(np.int64)
    bs = c.block_size
    first = np.zeros_like(L)
    if window > 0:
        first = np.maximum(L - window, 0)
    per_tok = 2 * c.n_kv_heads * c.head_dim * s_kv
    T = new_tokens
    total = int(((L - first - T) * per_tok).sum())               # read cached K, V
    total += wl.batch * T * per_tok                              # write new K, V
    total += wl.batch * T * (2 * c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim * s_io
    total += int((4 * ((L + bs - 1) // bs - first // bs) + 8).sum())
    total += wl.batch * T * c.head_dim * 4                       # cos + sin rows
    if c.kv_dtype == "fp8":
        total += 16 * c.n_kv_heads
    return total


def attention_flops(wl, window: int = 0, new_tokens: int = 1) -> int:
    """Multiply-adds of the step's attention, counted as 2 FLOPs each: the
    scores q.K and the weighted sum p.V, D each, for every query head and
    every token it attends to (the whole context, its last ``window`` tokens
    with a window, or causally the first L - T + i + 1 for new token i of T)."""
    c = wl.cfg
    L = wl.context_lens.astype(np.int64)
    T = new_tokens
    attended = np.zeros_like(L)
    for i in range(T):
        n = L - T + i + 1
        attended += np.minimum(n, window) if window > 0 else n
    return int(4 * c.n_q_heads * c.head_dim * attended.sum())


# Context from the pages (another GPU, another path: not a target): "TensorRT-LLM
# Guide: High-Throughput GPU Inference Engine", section "1. The Arithmetic
# Intensity Mismatch" puts a whole decode step near 1 FLOP per byte on an H100
# with 3.35 TB/s of HBM3 and nearly 1000 dense FP16 TFLOPS.
PAGES_CONTEXT = {"gpu": "H100 (the pages' example)", "hbm_TB_s": 3.35, "fp16_dense_TFLOPS": 1000,
                 "decode_step_flop_per_byte": 1.0}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("decode.hip", "plan.h", "kernels.h"):
        with open(os.path.join(ROOT, "paged_kv_decode_step_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, per_launch_alg: float):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def synth_pool_chunks(wl, device, chunk_blocks: int = 4096):
    """Cached K/V drawn on the device (float32 N(0,1), seeded per chunk) and
    cast to the cache type with torch's conversions: bf16 round-to-nearest,
    fp8 with per-head scales amax/448 and saturation.  Returns a generator of
    (first_block, k_codes, v_codes) in the logical layout, and the scales."""
    import torch
    import workloads

    c = wl.cfg
    nb = wl.num_blocks
    scales = None
    if c.kv_dtype == "fp8":
        amax = {"k_cache": torch.zeros(c.n_kv_heads, device=device),
                "v_cache": torch.zeros(c.n_kv_heads, device=device)}
        for b0 in range(0, nb, chunk_blocks):
            n = min(chunk_blocks, nb - b0)
            for w in amax:
                x = workloads.device_normals(wl, w, device, b0, n)
                amax[w] = torch.maximum(amax[w], x.abs().amax(dim=(0, 2, 3)))
                del x
        scales = tuple((amax[w] / 448.0).float().cpu().numpy() for w in ("k_cache", "v_cache"))

    def cast(x, i):
        if c.kv_dtype == "bf16":
            return x.to(torch.bfloat16).view(torch.int16)
        if c.kv_dtype == "f32":
            return x
        inv = torch.from_numpy(np.float32(1.0) / scales[i]).to(device)
        return (x * inv.view(1, -1, 1, 1)).clamp(-448.0, 448.0).to(
            torch.float8_e4m3fn).view(torch.uint8)

    def chunks():
        for b0 in range(0, nb, chunk_blocks):
            n = min(chunk_blocks, nb - b0)
            yield (b0, cast(workloads.device_normals(wl, "k_cache", device, b0, n), 0),
                   cast(workloads.device_normals(wl, "v_cache", device, b0, n), 1))

    return chunks, scales


def synth_io(wl, device):
    """q, k_new, v_new: host-drawn N(0,1) cast to the I/O dtype by torch."""
    import torch
    import workloads

    dt = torch.float32 if wl.cfg.io_dtype == "f32" else torch.bfloat16
    host = {w: workloads.host_normals(wl, w) for w in ("q", "k_new", "v_new")}
    return {w: torch.from_numpy(x).to(device).to(dt) for w, x in host.items()}


def setup_layers(wl, n_layers, device):
    """Pools filled with device-drawn values, plus the step's inputs."""
    import torch
    import paged_kv_decode_step_amd as pkv
    from paged_kv_decode_step_amd import pool_io

    c = wl.cfg
    chunks, scales = synth_pool_chunks(wl, device)
    pools = []
    for _ in range(n_layers):
        pool = pkv.KVPool(wl.num_blocks, c.block_size, c.n_kv_heads, c.head_dim, c.kv_dtype)
        pool.set_rope(c.rope_theta, wl.max_position)
        if scales is not None:
            pool.set_fp8_scales(*scales)
        pools.append(pool)
    for b0, k, v in chunks():
        for pool in pools:
            pool_io.write_logical(pool, k, v, b0)
        del k, v
    tens = synth_io(wl, device)
    tens["positions"] = torch.from_numpy(wl.positions.astype(np.int32)).to(device)
    tens["block_tables"] = torch.from_numpy(wl.block_tables.astype(np.int32)).to(device)
    tens["context_lens"] = torch.from_numpy(wl.context_lens.astype(np.int32)).to(device)
    tens["out"] = torch.empty_like(tens["q"])
    torch.cuda.synchronize()
    return pools, tens, scales


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def achievable_peak(device, n_bytes: int = 4 << 30, reps: int = 10,
                    step_bytes: int = 0) -> dict:
    """What a plain streaming read reaches on this GPU (pkv_stream_read: the
    attention kernel's 16-byte nontemporal loads, no arithmetic), timed with
    events: one large buffer read `reps` times, and, with `step_bytes` up to
    half of it, reads of `step_bytes` each, back to back, rotating over the
    buffer's disjoint regions (at least two, together far larger than the
    256 MB Infinity Cache) so that no read finds its data in a cache: the
    step's own bytes moved at the step's own size, with the launch, ramp and
    drain costs a step of that size meets."""
    import torch
    import paged_kv_decode_step_amd as pkv

    src = torch.empty(n_bytes, dtype=torch.uint8, device=device)
    sink = torch.zeros(256, dtype=torch.int32, device=device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(views, n):
        for v in views:
            pkv.stream_read(v, sink)
        torch.cuda.synchronize()
        e0.record()
        for k in range(n):
            pkv.stream_read(views[k % len(views)], sink)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms = timed([src], reps)
    gbs = n_bytes / (ms * 1e-3) / 1e9
    out = {"kernel": "pkv_stream_read (16-byte nontemporal loads, one pass)",
           "bytes": n_bytes, "ms": round(ms, 4), "GB/s": round(gbs, 1),
           "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4), "at_step_bytes": None}
    nb = step_bytes // 16 * 16
    if nb > 0 and 2 * nb <= n_bytes:
        views = [src[i * nb:(i + 1) * nb] for i in range(n_bytes // nb)]
        ms_s = timed(views, max(48, 2 * len(views)))
        gbs_s = nb / (ms_s * 1e-3) / 1e9
        out["at_step_bytes"] = {"bytes": nb, "regions": len(views), "us": round(ms_s * 1e3, 2),
                                "GB/s": round(gbs_s, 1), "frac_of_peak": round(gbs_s / PEAK_HBM_GBS, 4)}
    del src, sink
    torch.cuda.empty_cache()
    return out


def cpu_baseline(wl, pool, tens, scales, budget_s: float, window: int = 0):
    """Time the CPU oracle on leading requests of the workload until about
    `budget_s` seconds of work, reading their inputs back from the device."""
    import torch
    import oracle
    from paged_kv_decode_step_amd import pool_io
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import gpu_problem as gp

    def host_io(x):
        if x.dtype == torch.bfloat16:
            return x.view(torch.int16).cpu().numpy().view(np.uint16)
        return x.cpu().numpy()
    io = {w: host_io(tens[w]) for w in ("q", "k_new", "v_new")}

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        ncores = len(os.sched_getaffinity(0))
        limiter = threadpool_limits(ncores)
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: numpy's default
        limiter, threads = None, len(os.sched_getaffinity(0))
    c = wl.cfg
    elapsed, done_bytes, done_req, passes = 0.0, 0, 0, 0
    budget_hit = False
    # whole passes over the workload's requests (or the leading requests of
    # one pass) until the budget of CPU work is used
    while not budget_hit and passes < 1000:
        passes += 1
        for b in range(wl.batch):
            nblk = int(wl.n_blocks_used()[b])
            ids = torch.from_numpy(wl.block_tables[b, :nblk].astype(np.int64)).to(
                pool.k_storage().device)
            k, v = pool_io.gather_blocks_logical(pool, ids)
            kc, vc = gp.codes_from_torch(k, c.kv_dtype), gp.codes_from_torch(v, c.kv_dtype)
            mwl, arrs = gp.mini_problem(wl, b, kc, vc, io, scales)
            t0 = time.perf_counter()
            oracle.decode_step(k_pool=arrs["k_pool"], v_pool=arrs["v_pool"], kv_dtype=c.kv_dtype,
                               io_dtype=c.io_dtype, q=arrs["q"], k_new=arrs["k_new"],
                               v_new=arrs["v_new"], positions=mwl.positions,
                               block_tables=mwl.block_tables, context_lens=mwl.context_lens,
                               block_size=c.block_size, rope_theta=c.rope_theta,
                               k_scale=arrs["k_scale"], v_scale=arrs["v_scale"], window=window)
            elapsed += time.perf_counter() - t0
            done_bytes += algorithmic_bytes(mwl, window)
            done_req += 1
            if elapsed >= budget_s:
                budget_hit = True
                break
    if limiter is not None and hasattr(limiter, "unregister"):
        limiter.unregister()
    if passes == 1 and budget_hit:
        sample = f"the first {done_req} of {wl.batch} requests of the workload"
    else:
        sample = (f"{done_req} requests: {passes} passes over all {wl.batch} requests of the "
                  f"workload (the last one partial)")
    return {
        "value": round(done_bytes / elapsed / 1e9, 4), "unit": "GB/s",
        "tokens_per_s_per_layer": round(done_req / elapsed, 2),
        "cores": int(threads), "kind": "oracle", "cpu_model": cpu_model(),
        "sample": f"{sample}; {elapsed:.1f} s of numpy fp64 work (block gather, RoPE, append, "
                  f"attention per request; device-to-host transfer excluded)",
    }


def allocator_bench(wl, device, steps: int) -> dict:
    """Host cost of the allocator's step for the workload's batch (every
    request grows by one token; half of them forked from a parent so their
    half-full last blocks are copied on write), and the device copy of whole
    blocks: bytes = 2 (K and V) x 2 (read and write) x block bytes per pair."""
    import torch
    import paged_kv_decode_step_amd as pkv

    c = wl.cfg
    lens = wl.context_lens.astype(np.int64)
    nb = int(((lens + c.block_size) // c.block_size).sum()) * 2 + 16
    alloc = pkv.BlockAllocator(nb, c.block_size, 2 * wl.batch + 1)
    seqs = [alloc.add(int(L) - 1) for L in lens]
    reps, t_host = max(1, min(steps, 50)), 0.0
    maxb = int(wl.block_tables.shape[1]) + (reps + 2) // c.block_size + 2
    # the host arrays a serving loop keeps from step to step
    bufs = (np.empty((len(seqs), maxb), np.int32), np.empty(len(seqs), np.int32),
            np.empty(len(seqs), np.int32), np.empty((len(seqs), 2), np.int32))
    alloc.prepare_step(seqs, maxb, out=bufs)          # first touch of the host arrays
    for _ in range(reps):
        t0 = time.perf_counter()
        alloc.prepare_step(seqs, maxb, out=bufs)
        t_host += time.perf_counter() - t0
    # copy on write: fork every other request, then one step copies each
    # shared half-full block once
    kids = [alloc.fork(s) for s in seqs[::2]]
    _, _, _, copies = alloc.prepare_step(seqs[::2], maxb)
    alloc.close()
    pool = pkv.KVPool(nb, c.block_size, c.n_kv_heads, c.head_dim, c.kv_dtype)
    pairs = torch.from_numpy(np.ascontiguousarray(copies)).to(device)
    block_bytes = c.n_kv_heads * c.block_size * c.head_dim * ELEM[c.kv_dtype]
    for _ in range(3):
        pool.copy_blocks(pairs)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_rep = max(10, steps)
    e0.record()
    for _ in range(n_rep):
        pool.copy_blocks(pairs)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n_rep
    pool.close()
    moved = 4 * block_bytes * int(pairs.shape[0])
    return {"metric": "block allocator: host prepare_step us per decode step; device block "
                      "copy GB/s", "workload": c.name, "batch": wl.batch,
            "prepare_step_us": round(1e6 * t_host / reps, 2),
            "forked": len(kids), "copies": int(pairs.shape[0]),
            "copy_ms": round(ms, 5), "copy_GBps": round(moved / (ms * 1e-3) / 1e9, 2),
            "block_bytes": block_bytes}


def make_bench_workload(args):
    """The workload of ``--config``, or one GPU's head shard of it with
    ``--tp`` above 1."""
    import workloads
    if args.tp > 1:
        return workloads.shard_workload(args.config, args.tp)
    return workloads.make_workload(args.config)


def timeline_summary(rec) -> dict:
    """Where one step's attention kernel spent its time, from the
    per-wavefront records of ``kv_pool_read_timeline`` (stamps of a 100 MHz
    clock): when the wavefronts started (dispatch skew), how long each phase
    took (median over the wavefronts with tiles), when they finished, and the
    same per XCD.  Times in microseconds from the first wavefront's entry."""
    rec = np.asarray(rec, dtype=np.int64)
    t0 = rec[:, 0].min()
    us = (rec[:, :6] - t0) / 100.0
    tiles = rec[:, 6]
    xcc = (rec[:, 7] >> 32) & 0xF
    act = tiles > 0
    a, ta, xa = us[act], tiles[act], xcc[act]
    span = float(a[:, 5].max())
    pc = lambda v, q: round(float(np.percentile(v, q)), 2)
    med = lambda v: round(float(np.median(v)), 2)
    loop = a[:, 4] - a[:, 3]
    per_xcd = {}
    for x in np.unique(xa):
        m = xa == x
        per_xcd[int(x)] = {"waves": int(m.sum()), "start_p50": med(a[m, 0]),
                           "end_p50": med(a[m, 5]), "end_max": round(float(a[m, 5].max()), 2),
                           "tiles_per_us_p50": round(float(np.median(ta[m] / np.maximum(loop[m], 1e-3))), 3)}
    return {
        "waves": int(len(rec)), "active": int(act.sum()), "span_us": round(span, 2),
        "start_us": {"p50": pc(a[:, 0], 50), "p90": pc(a[:, 0], 90), "max": pc(a[:, 0], 100)},
        "phase_us_p50": {"request_table": med(a[:, 1] - a[:, 0]), "tile_range": med(a[:, 2] - a[:, 1]),
                         "ring_fill": med(a[:, 3] - a[:, 2]), "tile_loop": med(loop),
                         "writes_and_exit": med(a[:, 5] - a[:, 4])},
        "end_us": {"p10": pc(a[:, 5], 10), "p50": pc(a[:, 5], 50), "p90": pc(a[:, 5], 90),
                   "max": round(span, 2)},
        "busy_fraction": round(float((a[:, 5] - a[:, 0]).sum() / (len(a) * span)), 4),
        "tiles_p50": med(ta), "per_xcd": per_xcd,
    }


def timeline_bench(args) -> dict:
    """Run the timeline build of the library on the workload and summarise
    the per-wavefront records of a few steps, each launched right behind
    another step."""
    import torch
    import paged_kv_decode_step_amd as pkv
    import workloads

    pkv.load_library(pkv.TIMELINE_LIB_PATH)
    wl = make_bench_workload(args)
    pools, t, _ = setup_layers(wl, 1, "cuda:0")
    pool = pools[0]
    pool.set_window(args.window)
    T = args.new_tokens
    if T > 1:
        dt = t["q"].dtype
        gen = torch.Generator(device="cuda:0").manual_seed(1234)
        c = wl.cfg
        for w, h in (("q", c.n_q_heads), ("k_new", c.n_kv_heads), ("v_new", c.n_kv_heads)):
            t[w] = torch.randn(wl.batch, T, h, c.head_dim, device="cuda:0", generator=gen).to(dt)
        t["out"] = torch.empty_like(t["q"])
        t["positions"] = (t["context_lens"] - T).contiguous()

    def step():
        if T > 1:
            pkv.decode_step_multi(pool, t["q"], t["k_new"], t["v_new"], t["positions"],
                                  t["block_tables"], t["context_lens"], t["out"])
        else:
            pkv.decode_step(pool, t["q"], t["k_new"], t["v_new"], t["positions"],
                            t["block_tables"], t["context_lens"], t["out"])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    reps = []
    for _ in range(max(1, args.steps)):
        # two steps back to back: the records are the second's, a step
        # launched behind another as in a decode loop (reading them
        # synchronises, so a single step would start on an idle GPU)
        step()
        step()
        reps.append(timeline_summary(pool.read_timeline()))
    pool.close()
    return {"metric": "attention kernel per-wavefront timeline (timeline build)",
            "workload": wl.cfg.name, "window": args.window, "new_tokens": T,
            "span_us_p50": round(float(np.median([r["span_us"] for r in reps])), 2),
            "steps": reps}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=5,
                    help="workload 1..5 (default 5, the largest: 512 mixed-length requests, "
                         "15.5 GB of cache per step)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of CPU oracle work for the baseline (0 = skip)")
    ap.add_argument("--min-cold-bytes", type=float, default=1.0e9)
    ap.add_argument("--window", type=int, default=0,
                    help="sliding-window attention over the last W tokens (0 = whole context)")
    ap.add_argument("--new-tokens", type=int, default=1,
                    help="T new tokens per request (decode_step_multi; the lengths count them)")
    ap.add_argument("--tp", type=int, default=1,
                    help="measure one GPU's shard of the workload when its heads are split over "
                         "TP GPUs (Hkv/TP KV heads and their query heads, same requests); the "
                         "run itself stays on one GPU")
    ap.add_argument("--allocator", action="store_true",
                    help="only measure the block allocator's host step (prepare_step for the "
                         "workload's batch) and the device block copy, one JSON line")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay of the multi-layer step")
    ap.add_argument("--timeline", action="store_true",
                    help="run the timeline build of the library (libpkv_timeline.so) for "
                         "--steps single steps after --warmup and print the per-wavefront "
                         "phase summary of each, one JSON line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run --steps plain device copies of 1 GiB (for scaling "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    if args.timeline:
        print(json.dumps(timeline_bench(args)), flush=True)
        return

    import torch
    import paged_kv_decode_step_amd as pkv
    import workloads

    device = "cuda:0"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=device)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": args.steps}), flush=True)
        return
    wl = make_bench_workload(args)
    c = wl.cfg
    if args.allocator:
        print(json.dumps(allocator_bench(wl, device, args.steps)), flush=True)
        return
    alg = algorithmic_bytes(wl, args.window, args.new_tokens)
    kv_bytes = int(((wl.context_lens.astype(np.int64)) * 2 * c.n_kv_heads * c.head_dim
                    * ELEM[c.kv_dtype]).sum())
    n_layers = max(1, math.ceil(args.min_cold_bytes / (min(kv_bytes, alg) if args.window else kv_bytes)))
    pools, t, scales = setup_layers(wl, n_layers, device)
    for p in pools:
        p.set_window(args.window)
    print(f"# workload {c.name}: {wl.batch} requests, {alg/1e9:.3f} GB algorithmic per step, "
          f"{n_layers} pool copies, {pools[0].info()['n_waves']} wavefronts", file=sys.stderr,
          flush=True)

    T = args.new_tokens
    if T > 1:
        # T new tokens per request: [B, T, H, D] inputs; positions of the first new token
        dt = t["q"].dtype
        gen = torch.Generator(device=device).manual_seed(1234)
        for w, h in (("q", c.n_q_heads), ("k_new", c.n_kv_heads), ("v_new", c.n_kv_heads)):
            t[w] = torch.randn(wl.batch, T, h, c.head_dim, device=device, generator=gen).to(dt)
        t["out"] = torch.empty_like(t["q"])
        t["positions"] = (t["context_lens"] - T).contiguous()

    def step(i):
        if T > 1:
            pkv.decode_step_multi(pools[i % n_layers], t["q"], t["k_new"], t["v_new"],
                                  t["positions"], t["block_tables"], t["context_lens"], t["out"])
            return
        pkv.decode_step(pools[i % n_layers], t["q"], t["k_new"], t["v_new"], t["positions"],
                        t["block_tables"], t["context_lens"], t["out"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K steps, bracketed by synchronisation; the step events
    # are on the stream the kernels are launched on (torch's current stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # the same K steps again, each kernel launched with start/stop events
    # that its own dispatch stamps (kernel durations, for the roofline); a
    # pass of its own so that the event packets do not sit in the timed steps
    for p in pools:
        p.enable_timing(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    attn_ms = merge_ms = 0.0
    calls = 0
    for p in pools:
        a, m, n = p.read_timing()
        attn_ms, merge_ms, calls = attn_ms + a, merge_ms + m, calls + n
        p.enable_timing(False)
    attn_avg = attn_ms / max(calls, 1)
    merge_avg = merge_ms / max(calls, 1)

    # the same steps replayed from one HIP graph that records a step on every
    # pool copy: a multi-layer decode step issued with a single launch
    graph_ms, graph_error = None, None
    if not args.no_graph:
        try:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for i in range(n_layers):
                    step(i)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(n_layers):
                    step(i)
            reps = max(1, args.steps // n_layers)
            graph.replay()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            graph_ms = e0.elapsed_time(e1) / (reps * n_layers)
            del graph
        except Exception as exc:   # the graph figure is optional; the eager line stands
            graph_error = f"{type(exc).__name__}: {exc}"
            torch.cuda.synchronize()

    gbs = alg / (ms_per_step * 1e-3) / 1e9
    achieved = alg / (attn_avg * 1e-3) / 1e9
    traffic = measured_traffic(c.name, alg)
    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.kv_dtype if c.kv_dtype != "f32" else "f32",
        "data": "synthetic",
        "config": {"workload": c.name, "batch": wl.batch, "n_q_heads": c.n_q_heads,
                   "n_kv_heads": c.n_kv_heads, "head_dim": c.head_dim,
                   "block_size": c.block_size, "kv_dtype": c.kv_dtype,
                   "io_dtype": c.io_dtype, "mean_context": float(wl.context_lens.mean()),
                   "pool_copies": n_layers, "window": args.window,
                   "new_tokens": args.new_tokens, "tp_shard": args.tp},
        "pct_of_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "tokens_per_s_per_layer": round(wl.batch * T / (ms_per_step * 1e-3), 1),
        "algorithmic_bytes_per_step": alg,
        "kernel_ms": {"attention": round(attn_avg, 5), "merge": round(merge_avg, 5)},
        "graph": ({"error": graph_error} if graph_error else None) if graph_ms is None else {
            "layers": n_layers, "ms_per_step": round(graph_ms, 5),
            "GB/s": round(alg / (graph_ms * 1e-3) / 1e9, 2),
            "note": "one HIP graph replays a step on each pool copy (a multi-layer step); "
                    "value above is from eager launches"},
        "wall_s_timed_region": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic},
        "cpu_baseline": None,
        "achievable_peak": None,
        "context": dict(PAGES_CONTEXT, attention_flop_per_byte_here=round(
            attention_flops(wl, args.window, T) / alg, 3)),
    }
    # the other pool copies are freed before the 4 GiB streaming read; the
    # first one stays for the CPU baseline, which reads its blocks back
    for p in pools[1:]:
        p.close()
    result["achievable_peak"] = achievable_peak(device, step_bytes=alg)
    at = result["achievable_peak"]["at_step_bytes"]
    if at:   # the attention kernel against a plain read of the same bytes
        result["roofline"]["frac_of_plain_read_at_step_bytes"] = round(achieved / at["GB/s"], 4)
    if args.cpu_budget > 0 and T == 1:
        result["cpu_baseline"] = cpu_baseline(wl, pools[0], t, scales, args.cpu_budget,
                                              args.window)
    pools[0].close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
