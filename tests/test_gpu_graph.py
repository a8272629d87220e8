"""GPU: a multi-layer decode step (one pool per layer) captured as one HIP
graph.  CUDA graphs remove launch overhead by replaying a recorded sequence
of launches ("Lesson 13.17 TensorRT-LLM: NVIDIA's Optimized Inference
Engine", section "The paged KV cache, in-flight batching and CUDA graphs");
decode_step allocates nothing and never synchronises, so its launches can be
recorded.  Every replay, with eager work and synchronisations between
replays, must give the eager outputs and pools bit for bit, and those match
the oracle."""
import numpy as np
import pytest
import torch

import gpu_problem as gp
import paged_kv_decode_step_amd as pkv
import problem
import workloads

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_multi_layer_step_replayed_from_a_graph(kv):
    lens = [1, 37, 200, 513, 1000, 64]
    runs, refs = [], []
    for layer in range(3):
        wl = workloads.custom_workload(lens, n_q_heads=16, n_kv_heads=4, head_dim=128,
                                       block_size=16 if kv == "bf16" else 32, kv_dtype=kv,
                                       io_dtype="bf16", rope_theta=5.0e5, seed=40 + layer)
        arrs = problem.build(wl)
        refs.append(problem.oracle_step(wl, arrs))
        runs.append(gp.Run(wl, arrs))

    def launch(r):
        pkv.decode_step(r.pool, r.q, r.k_new, r.v_new, r.positions, r.tables, r.lens, r.out)

    try:
        for r in runs:
            r.step()
        eager_out = [r.out.clone() for r in runs]
        eager_pools = [r.pools() for r in runs]
        for r, ref in zip(runs, refs):
            assert gp.row_rel_err(r.out_f64(), ref["out"]).max() <= gp.tolerance(kv)
            kp, vp = r.pools()
            assert np.array_equal(gp.bits(kp), gp.bits(ref["k_pool"]))
            assert np.array_equal(gp.bits(vp), gp.bits(ref["v_pool"]))

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for r in runs:
                launch(r)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in runs:
                launch(r)
        for rep in range(3):
            for r in runs:
                r.out.fill_(float("nan"))
            # eager work of the program's own between replays
            x = torch.randn(256, 256, device=gp.DEV)
            (x @ x).sum().item()
            runs[rep % len(runs)].step()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for r, eo, (ek, ev) in zip(runs, eager_out, eager_pools):
                assert torch.equal(r.out.view(torch.int16), eo.view(torch.int16)), rep
                kp, vp = r.pools()
                assert np.array_equal(gp.bits(kp), gp.bits(ek)) and np.array_equal(gp.bits(vp), gp.bits(ev))
        for r in runs:
            assert r.pool.device_errors() == 0
    finally:
        for r in runs:
            r.close()


@pytest.mark.parametrize("mode", ["window", "multi"])
def test_windowed_and_multi_token_steps_replay_from_a_graph(mode):
    """The windowed step and the multi-token step (its append launch, the
    attention and the merge) record into a graph too; every replay gives the
    eager outputs and pools bit for bit."""
    lens = [5, 37, 200, 513, 1000]
    wl = workloads.custom_workload(lens, n_q_heads=16, n_kv_heads=4, head_dim=128, block_size=16,
                                   kv_dtype="bf16", io_dtype="bf16", rope_theta=5.0e5, seed=77)
    arrs = problem.build(wl)
    run = gp.Run(wl, arrs, max_position=2048)
    try:
        rng = np.random.default_rng(77)
        if mode == "window":
            run.pool.set_window(100)

            def launch():
                pkv.decode_step(run.pool, run.q, run.k_new, run.v_new, run.positions, run.tables,
                                run.lens, run.out)
            out = run.out
        else:
            tq, b = 3, len(lens)
            enc = lambda shape: gp.io_to_torch(
                problem.encode_io(rng.standard_normal(shape).astype(np.float32), "bf16"), "bf16")
            q, kn, vn = enc((b, tq, 16, 128)), enc((b, tq, 4, 128)), enc((b, tq, 4, 128))
            pos = (run.lens - tq).contiguous()
            out = torch.full_like(q, float("nan"))

            def launch():
                pkv.decode_step_multi(run.pool, q, kn, vn, pos, run.tables, run.lens, out)
        launch()
        torch.cuda.synchronize()
        eager_out = out.clone()
        eager_pools = run.pools()
        assert torch.isfinite(eager_out.float()).all()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            launch()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            launch()
        for rep in range(3):
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), eager_out.view(torch.int16)), rep
            kp, vp = run.pools()
            assert np.array_equal(gp.bits(kp), gp.bits(eager_pools[0]))
            assert np.array_equal(gp.bits(vp), gp.bits(eager_pools[1]))
        assert run.pool.device_errors() == 0
    finally:
        run.close()
