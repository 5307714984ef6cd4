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
    ("moe_b1", dict(n_layers=1, vocab=8192)),
    ("moe_b32", dict(n_layers=2, vocab=4096, batch=20, ctx=("uniform", 50, 400))),
])
def test_graph_replays_match_eager(H, name, overrides):
    cfg = workloads.scaled(workloads.get_config(name), **overrides)
    case = H.Case(cfg)
    run = H.GpuRun(case, debug=False)
    H.say(f"[graph {name}] B={run.B} L={cfg.n_layers}")
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
