"""The verify step captured into a HIP graph (torch.cuda.CUDAGraph): every
replay, with eager work and synchronisations between replays, must give the
eager step's outputs bit for bit (the step enqueues kernels only: no host
synchronisation, no memset nodes).  Covers the few-row path (batch 1: fused
QKV, implied routing) and the many-row path (permutation kernel, large-row
GEMMs)."""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_harness
    return gpu_harness


@pytest.mark.parametrize("name,overrides", [
    ("moe_b1", {}),       # the full-size batch-1 workload, as bench.py replays it
    ("moe_b1", dict(n_layers=1, vocab=8192)),
    ("moe_b32", dict(n_layers=2, vocab=4096, batch=20, ctx=("uniform", 50, 400))),
])
def test_graph_replays_match_eager(H, name, overrides):
    cfg = workloads.scaled(workloads.get_config(name), **overrides) if overrides else \
        workloads.get_config(name)
    case = H.Case(cfg)
    run = H.GpuRun(case, debug=False)
    H.say(f"[graph {name}] B={run.B} L={cfg.n_layers} V={cfg.vocab}")
    dev = "cuda"
    com = case.committed[: run.B].to(dev, torch.int32).contiguous()
    dr = case.rtok[0][: run.B].to(dev, torch.int32).contiguous()
    ci = case.ctx[: run.B].to(dev, torch.int32).contiguous()
    co = torch.full((run.B,), -9, dtype=torch.int32, device=dev)

    def step():
        run.ctx.step(run.kc, run.vc, com, dr, ci, co, run.acc, run.nxt, batch=run.B)

    step()
    torch.cuda.synchronize()
    eager = (run.acc.clone(), run.nxt.clone(), co.clone())

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        run.acc.fill_(-1)
        run.nxt.fill_(-1)
        co.fill_(-1)
        _ = torch.ones(1024, device=dev).sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want, nm in zip((run.acc, run.nxt, co), eager, ("accepted", "next_tok", "ctx_out")):
            assert torch.equal(got, want), f"replay {rep}: {nm}"
    assert run.ctx.error_word() == 0
    run.close()


@pytest.mark.parametrize("name,overrides", [
    ("moe_b1", {}),       # the full-size batch-1 workload, as bench.py replays it
    ("moe_b1", dict(n_layers=1, vocab=8192)),
    ("dense_fp8_b8", dict(n_layers=1, vocab=8192, batch=3, k_draft=7, ctx=("uniform", 100, 300))),
])
def test_sampled_graph_replays_match_eager(H, name, overrides):
    """The sampled step (statistics, decision + draw, commit) captured the
    same way: replays equal the eager step for the same seed and offset."""
    cfg = workloads.scaled(workloads.get_config(name), **overrides)
    case = H.Case(cfg)
    run = H.GpuRun(case, debug=False)
    sd = workloads.sampled_drafts(cfg)
    H.say(f"[sampled graph {name}] B={run.B} L={cfg.n_layers} K={cfg.k_draft}")
    dev = "cuda"
    com = case.committed[: run.B].to(dev, torch.int32).contiguous()
    dr = sd["drafts"][: run.B].to(dev).contiguous()
    q = sd["q"][: run.B].to(dev).contiguous()
    u = sd["u"][: run.B].to(dev).contiguous()
    ci = case.ctx[: run.B].to(dev, torch.int32).contiguous()
    co = torch.full((run.B,), -9, dtype=torch.int32, device=dev)

    def step():
        run.ctx.step_sampled(run.kc, run.vc, com, dr, q, u, 0.9, sd["seed"], 5, ci, co, run.acc,
                             run.nxt, batch=run.B)

    step()
    torch.cuda.synchronize()
    eager = (run.acc.clone(), run.nxt.clone(), co.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        run.acc.fill_(-1)
        run.nxt.fill_(-1)
        co.fill_(-1)
        _ = torch.ones(1024, device=dev).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want, nm in zip((run.acc, run.nxt, co), eager, ("accepted", "next_tok", "ctx_out")):
            assert torch.equal(got, want), f"replay {rep}: {nm}"
    assert run.ctx.error_word() == 0
    run.close()
