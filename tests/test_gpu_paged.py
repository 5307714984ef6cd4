"""Paged KV caches (spec_verify_set_kv_pages): the same step on caches split
into pages of a shuffled pool must give the contiguous step's results bit for
bit (the kernels only read and write different addresses, in the same order)
and must match the oracle on its natural caches under the parity rules;
sequences sharing the pages of a common prefix must match unshared copies and
the oracle; a page index outside the pool is reported, not followed; and a
chain of steps captured into one HIP graph replays like the eager chain."""
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


def _unpage(pool, table, B, cap, page):
    """Pool [n_pages][L][n_kv][page][D] + table -> contiguous [B][L][n_kv][cap][D]."""
    npg = cap // page
    idx = table.reshape(-1).long()
    p = pool[idx].reshape(B, npg, *pool.shape[1:])            # [B][npg][L][n_kv][page][D]
    return p.permute(0, 2, 3, 1, 4, 5).reshape(B, pool.shape[1], pool.shape[2], cap, pool.shape[4])


def _paged_run(H, case, B, page, order, committed, drafts, ctx, n_pool=None):
    import speculative_decoding_verify_step_amd as sv
    cfg = case.cfg
    kc, vc = sv.kv_to_library(case.k_nat[:B], case.v_nat[:B])
    kp, vp, table = sv.kv_paged_from_library(kc, vc, page, order)
    n_pool = kp.shape[0] if n_pool is None else n_pool
    ctx_obj = sv.VerifyContext(cfg, B, case.cap, case.w_gpu, kv_page_size=page, kv_pool_pages=n_pool)
    ctx_obj.set_kv_pages(table)
    dev = "cuda"
    i32 = dict(dtype=torch.int32, device=dev)
    K1, T = cfg.k_draft + 1, B * (cfg.k_draft + 1)
    logits = torch.full((B, K1, cfg.vocab), float("nan"), device=dev)
    target = torch.full((B, K1), -7, **i32)
    moe = cfg.ffn == "moe"
    routing = torch.full((cfg.n_layers, T, cfg.top_k), -1, **i32) if moe else None
    rlogits = torch.full((cfg.n_layers, T, cfg.n_experts), float("nan"), device=dev) if moe else None
    ctx_obj.set_debug(logits, None, target, routing)
    if moe:
        ctx_obj.set_debug_router(rlogits)
    acc, nxt, co = (torch.full((B,), -9, **i32) for _ in range(3))
    ctx_obj.step(kp, vp, committed.to(**i32), drafts.to(**i32).contiguous(), ctx.to(**i32), co,
                 acc, nxt)
    torch.cuda.synchronize()
    gd = {"accepted": acc.cpu().numpy(), "next_tok": nxt.cpu().numpy(), "ctx_out": co.cpu().numpy(),
          "target": target.cpu().numpy(), "logits": logits.cpu().numpy(), "hidden": None,
          "routing": routing.cpu().numpy() if moe else None,
          "rlogits": rlogits.cpu().numpy() if moe else None}
    return ctx_obj, kp, vp, table, acc.cpu(), nxt.cpu(), co.cpu(), logits.cpu(), gd


def _oracle_check(H, case, gd, seqs, committed, drafts, ctx, label):
    """The paged run's sequences `seqs` against the oracle on the natural
    caches (the parity rules of gpu_harness; the oracle follows the GPU's
    routing where it is a measured near-tie)."""
    cfg = case.cfg
    K1 = cfg.k_draft + 1
    orc = case.oracle()
    stats = {}
    for b in seqs:
        kc, vc = case.oracle_kv(b)
        forced = gd["routing"][:, b * K1:(b + 1) * K1][None] if gd["routing"] is not None else None
        o = orc.verify_step(kc, vc, [int(committed[b])], drafts[b:b + 1].numpy(), [int(ctx[b])],
                            want_logits=True, force_sel=forced, want_routing=forced is not None)
        if forced is not None:
            H.check_routing(cfg, forced, o, stats, label=f"{label} seq {b}",
                            rl_gpu=gd["rlogits"][:, b * K1:(b + 1) * K1])
        H.compare_sequence(cfg, gd, b, o, 0, stats, check_hidden=False)
    H.say(f"[{label}] oracle stats {stats}")
    if cfg.ffn == "moe":
        H.assert_forced_cap(stats, label)
    return stats


def _case(H, cfg, page):
    """A case whose cache capacity is a whole number of pages."""
    cap = (workloads.capacity_for(cfg) + page - 1) // page * page
    return H.Case(cfg, capacity=cap)


@pytest.mark.parametrize("name,overrides,page", [
    ("moe_b1", {}, 64),
    ("tiny_fp32", {"batch": 3, "ctx": ("uniform", 20, 400)}, 64),
    ("moe_b32", {"n_layers": 2, "vocab": 8192, "batch": 6, "ctx": ("uniform", 30, 700)}, 128),
    ("dense_fp8_b8", {"n_layers": 1, "vocab": 8192, "batch": 3, "k_draft": 7,
                      "ctx": ("uniform", 100, 500)}, 256),
    ("moe_b32", {"n_layers": 1, "vocab": 4096, "batch": 20, "ctx": ("uniform", 30, 300)}, 64),
])
def test_paged_equals_contiguous(H, name, overrides, page):
    cfg = workloads.scaled(workloads.get_config(name), **overrides) if overrides else \
        workloads.get_config(name)
    case = _case(H, cfg, page)
    B = cfg.batch
    checked = sorted({0, B - 1})
    drafts = case.drafts(checked)[:B]       # oracle drafts for the checked sequences
    run = H.GpuRun(case, batch=B)
    g = run.step(case.committed[:B], drafts, case.ctx[:B])
    npg = case.cap // page
    rng = np.random.default_rng(page + B)
    order = rng.permutation(B * npg)
    H.say(f"[paged {cfg.name}] B={B} cap={case.cap} page={page} pool={B * npg}")
    ctx_obj, kp, vp, table, acc, nxt, co, logits, gd = _paged_run(
        H, case, B, page, order, case.committed[:B], drafts, case.ctx[:B])
    assert ctx_obj.error_word() == 0
    _oracle_check(H, case, gd, checked, case.committed[:B], drafts, case.ctx[:B],
                  f"paged {cfg.name} vs oracle")
    assert np.array_equal(acc.numpy(), g["accepted"]) and np.array_equal(nxt.numpy(), g["next_tok"])
    assert np.array_equal(co.numpy(), g["ctx_out"])
    assert torch.equal(logits, torch.from_numpy(g["logits"]))
    kc2 = _unpage(kp, table, B, case.cap, page)
    vc2 = _unpage(vp, table, B, case.cap, page)
    assert torch.equal(kc2, run.kc) and torch.equal(vc2, run.vc)
    ctx_obj.close()
    run.close()


@pytest.mark.parametrize("name,overrides", [
    ("moe_b32", {"n_layers": 2, "vocab": 8192, "batch": 5, "ctx": ("uniform", 30, 700)}),
    ("moe_b1_mxfp4", {"n_layers": 1, "batch": 3, "ctx": ("uniform", 100, 900)}),
])
def test_paged_sampled_and_mxfp4_equal_contiguous(H, name, overrides):
    """The sampled step (rejection sampling, temperature 0.8) and MXFP4
    weights on paged caches in a shuffled pool: accepted lengths, tokens,
    contexts and the written pages equal the contiguous run's bit for bit."""
    import speculative_decoding_verify_step_amd as sv
    page = 64
    cfg = workloads.scaled(workloads.get_config(name), **overrides)
    case = _case(H, cfg, page)
    B = cfg.batch
    sd = workloads.sampled_drafts(cfg)
    dev = "cuda"
    i32 = dict(dtype=torch.int32, device=dev)
    com = case.committed[:B].to(**i32)
    dr = sd["drafts"].to(dev).contiguous()
    q, u = sd["q"].to(dev).contiguous(), sd["u"].to(dev).contiguous()
    ci = case.ctx[:B].to(**i32)
    npg = case.cap // page
    H.say(f"[paged sampled {cfg.name}] B={B} cap={case.cap} pool={B * npg}")
    outs = []
    for paged in (False, True):
        kc, vc = sv.kv_to_library(case.k_nat[:B], case.v_nat[:B])
        table = None
        if paged:
            kc, vc, table = sv.kv_paged_from_library(
                kc, vc, page, np.random.default_rng(7).permutation(B * npg))
        ctx_obj = sv.VerifyContext(cfg, B, case.cap, case.w_gpu, kv_page_size=page if paged else 0,
                                   kv_pool_pages=kc.shape[0] if paged else 0)
        if paged:
            ctx_obj.set_kv_pages(table)
        acc, nxt, co = (torch.full((B,), -9, **i32) for _ in range(3))
        ctx_obj.step_sampled(kc, vc, com, dr, q, u, 0.8, sd["seed"], sd["offset"], ci, co, acc, nxt)
        torch.cuda.synchronize()
        assert ctx_obj.error_word() == 0
        if paged:
            kc, vc = _unpage(kc, table, B, case.cap, page), _unpage(vc, table, B, case.cap, page)
        outs.append([acc.cpu(), nxt.cpu(), co.cpu(), kc, vc])
        ctx_obj.close()
    for got, want in zip(outs[1], outs[0]):
        assert torch.equal(got, want)


def test_paged_prefix_sharing(H):
    """Sequences 1..3 read sequence 0's pages for a common prefix of 4 pages;
    the results equal a contiguous run in which they hold copies of it."""
    import speculative_decoding_verify_step_amd as sv
    page = 64
    cfg = workloads.scaled(workloads.get_config("moe_b32"), n_layers=2, vocab=8192, batch=4,
                           ctx=("uniform", 300, 600))
    case = _case(H, cfg, page)
    B, pre = 4, 4 * page
    for b in range(1, B):   # give every sequence sequence 0's first `pre` positions
        case.k_nat[b, :, :, :pre] = case.k_nat[0, :, :, :pre]
        case.v_nat[b, :, :, :pre] = case.v_nat[0, :, :, :pre]
    drafts = case.drafts(range(B))[:B]
    run = H.GpuRun(case, batch=B)
    g = run.step(case.committed[:B], drafts, case.ctx[:B])
    npg = case.cap // page
    kc, vc = sv.kv_to_library(case.k_nat[:B], case.v_nat[:B])
    kp, vp, table = sv.kv_paged_from_library(kc, vc, page)
    table = table.clone()
    table[1:, :4] = table[0, :4]             # shared prefix pages
    ctx_obj = sv.VerifyContext(cfg, B, case.cap, case.w_gpu, kv_page_size=page,
                               kv_pool_pages=B * npg)
    ctx_obj.set_kv_pages(table)
    i32 = dict(dtype=torch.int32, device="cuda")
    K1, T = cfg.k_draft + 1, B * (cfg.k_draft + 1)
    logits = torch.full((B, K1, cfg.vocab), float("nan"), device="cuda")
    target = torch.full((B, K1), -7, **i32)
    routing = torch.full((cfg.n_layers, T, cfg.top_k), -1, **i32)
    rlogits = torch.full((cfg.n_layers, T, cfg.n_experts), float("nan"), device="cuda")
    ctx_obj.set_debug(logits, None, target, routing)
    ctx_obj.set_debug_router(rlogits)
    acc, nxt, co = (torch.full((B,), -9, **i32) for _ in range(3))
    ctx_obj.step(kp, vp, case.committed[:B].to(**i32), drafts.to(**i32).contiguous(),
                 case.ctx[:B].to(**i32), co, acc, nxt)
    torch.cuda.synchronize()
    assert ctx_obj.error_word() == 0
    assert np.array_equal(acc.cpu().numpy(), g["accepted"])
    assert np.array_equal(nxt.cpu().numpy(), g["next_tok"])
    assert torch.equal(logits.cpu(), torch.from_numpy(g["logits"]))
    gd = {"accepted": acc.cpu().numpy(), "next_tok": nxt.cpu().numpy(), "ctx_out": co.cpu().numpy(),
          "target": target.cpu().numpy(), "logits": logits.cpu().numpy(), "hidden": None,
          "routing": routing.cpu().numpy(), "rlogits": rlogits.cpu().numpy()}
    # every sequence against the oracle on natural caches holding the shared prefix
    _oracle_check(H, case, gd, range(B), case.committed[:B], drafts, case.ctx[:B],
                  "paged prefix vs oracle")
    ctx_obj.close()
    run.close()


def test_paged_bad_page_is_reported(H):
    import speculative_decoding_verify_step_amd as sv
    page = 64
    cfg = workloads.scaled(workloads.get_config("tiny_fp32"), batch=2, ctx=("fixed", 200))
    case = _case(H, cfg, page)
    B = 2
    kc, vc = sv.kv_to_library(case.k_nat[:B], case.v_nat[:B])
    kp, vp, table = sv.kv_paged_from_library(kc, vc, page)
    table = table.clone()
    table[1, 1] = 10 ** 6                    # a page the step reads, outside the pool
    ctx_obj = sv.VerifyContext(cfg, B, case.cap, case.w_gpu, kv_page_size=page,
                               kv_pool_pages=kp.shape[0])
    ctx_obj.set_kv_pages(table)
    i32 = dict(dtype=torch.int32, device="cuda")
    acc, nxt, co = (torch.full((B,), -9, **i32) for _ in range(3))
    ctx_obj.step(kp, vp, case.committed[:B].to(**i32), case.rtok[0][:B].to(**i32).contiguous(),
                 case.ctx[:B].to(**i32), co, acc, nxt)
    torch.cuda.synchronize()
    assert ctx_obj.error_word(clear=True) & sv.SV_DEV_CAPACITY
    ctx_obj.close()
    run = H.GpuRun(case, batch=B)
    with pytest.raises(sv.SpecVerifyError):   # a context without paged caches refuses a table
        sv.spec_verify_set_kv_pages(run.ctx.handle, table)
    run.close()


def test_paged_chain_replays_from_one_graph(H):
    """Six chained steps (contexts grow by accepted + 1, the bonus token is the
    next committed token, drafts from a fixed stream) captured into one HIP
    graph over paged caches: every replay from the restored start state gives
    the eager chain's accepted lengths, tokens and contexts."""
    import speculative_decoding_verify_step_amd as sv
    page, S = 64, 6
    cfg = workloads.scaled(workloads.get_config("moe_b1"), n_layers=1, vocab=8192, batch=4,
                           steps=S, ctx=("uniform", 100, 300))
    case = _case(H, cfg, page)
    B = cfg.batch
    kc, vc = sv.kv_to_library(case.k_nat[:B], case.v_nat[:B])
    kp0, vp0, table = sv.kv_paged_from_library(kc, vc, page, np.random.default_rng(3).permutation(
        B * (case.cap // page)))
    kp, vp = kp0.clone(), vp0.clone()
    ctx_obj = sv.VerifyContext(cfg, B, case.cap, case.w_gpu, kv_page_size=page,
                               kv_pool_pages=kp.shape[0])
    ctx_obj.set_kv_pages(table)
    i32 = dict(dtype=torch.int32, device="cuda")
    drafts = [case.rtok[s][:B].to(**i32).contiguous() for s in range(S)]
    com0 = case.committed[:B].to(**i32)
    ctx0 = case.ctx[:B].to(**i32)
    coms = [torch.empty(B, **i32) for _ in range(S + 1)]
    ctxs = [torch.empty(B, **i32) for _ in range(S + 1)]
    accs = [torch.empty(B, **i32) for _ in range(S)]

    def chain():
        for s_ in range(S):
            ctx_obj.step(kp, vp, coms[s_], drafts[s_], ctxs[s_], ctxs[s_ + 1], accs[s_], coms[s_ + 1])

    def restore():
        kp.copy_(kp0)
        vp.copy_(vp0)
        coms[0].copy_(com0)
        ctxs[0].copy_(ctx0)

    restore()
    chain()
    torch.cuda.synchronize()
    eager = [t.clone() for t in accs + coms + ctxs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        restore()
        chain()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        chain()
    for rep in range(3):
        restore()
        for t in accs + coms[1:] + ctxs[1:]:
            t.fill_(-1)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for got, want in zip(accs + coms + ctxs, eager):
            assert torch.equal(got, want), f"replay {rep}"
    assert ctx_obj.error_word() == 0
    grown = (ctxs[S] - ctxs[0]).cpu().numpy()
    assert np.all(grown >= S)                # every step commits at least the bonus token
    ctx_obj.close()
