"""Parity at the workloads' full sizes, in the configuration the benchmark
times (whole batch on one context, tiled16 weights), on sampled sequences the
oracle recomputes one by one.  The other sequences run with drafts from the
fallback tokens; every sequence's commit is still checked for consistency."""
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


def _run(H, name, sampled, steps=1):
    cfg = workloads.get_config(name)
    case = H.Case(cfg)
    B, K = cfg.batch, cfg.k_draft
    H.say(f"[full {name}] B={B} L={cfg.n_layers} V={cfg.vocab} K={K} cap={case.cap} "
          f"sampled={sampled} steps={steps}")
    run = H.GpuRun(case)
    orc = case.oracle()
    kv = {b: case.oracle_kv(b) for b in sampled}
    com = case.committed.clone()
    ctx_cpu = case.ctx.clone()
    ctx_dev = case.ctx.to("cuda", torch.int32).clone()
    coins, rtok = workloads.draft_randomness(cfg, steps=steps)
    stats = {}
    for s in range(steps):
        drafts = rtok[s].clone()
        for b in sampled:
            kc, vc = kv[b]
            drafts[b] = torch.from_numpy(orc.make_drafts(kc, vc, 0, int(ctx_cpu[b]), int(com[b]),
                                                         coins[s, b], rtok[s, b]))
        H.say(f"[full {name}] step {s}: drafts ready, GPU step")
        g = run.step(com, drafts, ctx_dev, ctx_out=ctx_dev)
        acc = g["accepted"]
        assert np.all((acc >= 0) & (acc <= K)), "every sequence commits 0..K drafts"
        assert np.array_equal(g["ctx_out"], ctx_cpu.numpy() + acc + 1)
        for b in sampled:
            kc, vc = kv[b]
            forced = run.routing_of(g, b)
            H.say(f"[full {name}] step {s}: oracle on sequence {b} (ctx {int(ctx_cpu[b])})")
            o = orc.verify_step(kc, vc, [int(com[b])], drafts[b:b + 1].numpy(), [int(ctx_cpu[b])],
                                want_logits=True, want_layer_hidden=True, force_sel=forced,
                                want_routing=forced is not None)
            H.check_routing(cfg, forced, o, stats, label=f"seq {b}")
            H.compare_sequence(cfg, g, b, o, 0, stats)
            if s == 0:
                H.compare_new_kv(cfg, run, b, kc, vc, int(ctx_cpu[b]), stats)
        # both sides continue from the GPU's commit (identical wherever checked)
        com = torch.from_numpy(g["next_tok"].copy())
        ctx_cpu = torch.from_numpy(g["ctx_out"].copy())
        for b in sampled:
            assert int(com[b]) >= 0
    H.say(f"[full {name}] stats {stats}")
    run.close()
    return stats


def test_full_size_moe_batch32(H):
    _run(H, "moe_b32", sampled=[0, 17])


def test_full_size_dense_fp8_k31(H):
    _run(H, "dense_fp8_b8", sampled=[3])


def test_full_size_moe_batch64_chained(H):
    _run(H, "moe_b64_long", sampled=[5, 40], steps=2)


def test_full_size_sampled_moe_batch64(H):
    """The sampled step at the batch-64 long-context workload's full size, in
    the configuration the benchmark times: the outcome of every sequence
    against the oracle's sampling on the GPU's logits, and two sequences'
    logits against the oracle's own forward."""
    from oracle import sampling as S
    cfg = workloads.get_config("moe_b64_long")
    case = H.Case(cfg)
    B, K = cfg.batch, cfg.k_draft
    sd = workloads.sampled_drafts(cfg)
    H.say(f"[full sampled] B={B} L={cfg.n_layers} V={cfg.vocab} cap={case.cap}")
    run = H.GpuRun(case)
    dev = "cuda"
    com = case.committed.to(dev, torch.int32).contiguous()
    ci = case.ctx.to(dev, torch.int32).contiguous()
    run.ctx.step_sampled(run.kc, run.vc, com, sd["drafts"].to(dev).contiguous(),
                         sd["q"].to(dev).contiguous(), sd["u"].to(dev).contiguous(), 1.0,
                         sd["seed"], sd["offset"], ci, run.ctx_out, run.acc, run.nxt, batch=B)
    torch.cuda.synchronize()
    ga, gn, gc = run.acc.cpu().numpy(), run.nxt.cpu().numpy(), run.ctx_out.cpu().numpy()
    assert run.ctx.error_word(clear=True) == 0
    glog = run.logits.cpu().double().numpy()
    o = S.sampled_verify(glog, sd["drafts"].numpy(), sd["q"].numpy(), sd["u"].numpy(), 1.0,
                         sd["seed"], sd["offset"], delta=1e-4, key_slack=1e-4)
    sure = o["accept_certain"] & o["draw_certain"]
    H.say(f"[full sampled] certain {int(sure.sum())}/{B}; accepted {ga[:8].tolist()}")
    assert sure.mean() >= 0.9
    for b in np.nonzero(sure)[0]:
        assert ga[b] == o["accepted"][b] and gn[b] == o["next_tok"][b]
        assert gc[b] == int(case.ctx[b]) + ga[b] + 1
    orc = case.oracle()
    tol = H.TOL[cfg.wdtype]
    stats = {}
    for b in (7, 50):
        kc, vc = case.oracle_kv(b)
        K1 = K + 1
        forced = run.routing.cpu().numpy()[:, b * K1:(b + 1) * K1][None]
        H.say(f"[full sampled] oracle forward of sequence {b} (ctx {int(case.ctx[b])})")
        ob = orc.verify_step(kc, vc, [int(case.committed[b])], sd["drafts"][b:b + 1].numpy(),
                             [int(case.ctx[b])], want_logits=True, force_sel=forced,
                             want_routing=True)
        H.check_routing(cfg, forced, ob, stats, label=f"seq {b}")
        for j in range(K1):
            lo = ob["logits"][0, j]
            err = float(np.abs(glog[b, j] - lo).max())
            assert err <= tol * float(lo.max() - lo.min()), f"seq {b} pos {j}: logits"
    run.close()
