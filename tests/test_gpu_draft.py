"""FastMTP drafting on the GPU (spec_draft_step) against the oracle
(Oracle.mtp_draft), after a GPU verify step.

Both sides start from the GPU verify step's outcome (accepted length, bonus
token) and from the same post-norm states: the oracle normalises the GPU's
last-layer residual rows in fp64 (the GPU's own states are those rows
normalised and rounded to the activation type).  A draft of depth k must equal
the oracle's wherever every depth up to k has an oracle top-2 logit gap above
the workload tolerance (2e-2 of the logit range for bf16 weights, 5e-2 for
fp8, 1e-4 for fp32): a near-tie there is a decision both answers of which are
correct to the arithmetic's precision, and later depths then start from
different tokens.  The block's cache rows written at the committed positions
are compared under the same tolerance.
"""
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


def _cpu(d):
    if isinstance(d, dict):
        return {k: _cpu(v) for k, v in d.items()}
    if isinstance(d, list):
        return [_cpu(v) for v in d]
    return d.cpu() if isinstance(d, torch.Tensor) else d


def _draft_case(H, cfg, label, min_checked=0.5):
    import oracle
    import speculative_decoding_verify_step_amd as sv
    case = H.Case(cfg)
    B, K = cfg.batch, cfg.k_draft
    K1 = K + 1
    drafts = case.drafts(list(range(B)))
    run = H.GpuRun(case, batch=B)
    g = run.step(case.committed[:B], drafts[:B], case.ctx[:B])
    H.say(f"[{label}] verify accepted {g['accepted'][:8].tolist()}")
    mc = workloads.mtp_config(cfg)
    mw = workloads.mtp_weights(cfg, "cuda")
    cap_m = (int(case.ctx[:B].max()) + 3 * K1 + 63) // 64 * 64
    mk, mv = workloads.kv_cache(workloads.scaled(mc, batch=B), "cuda", capacity=cap_m)
    mkl, mvl = sv.kv_to_library(mk, mv)
    dctx = sv.DraftContext(mc, B, cap_m, run.ctx.weights, mw)
    dev = "cuda"
    i32 = dict(dtype=torch.int32, device=dev)
    out = torch.full((B, K), -9, **i32)
    dctx.draft(mkl, mvl, run.ctx, case.ctx[:B].to(**i32), run.acc, run.nxt,
               drafts[:B].to(**i32).contiguous(), out)
    torch.cuda.synchronize()
    assert dctx.error_word(clear=True) == 0
    got = out.cpu().numpy()
    H.say(f"[{label}] gpu drafts {got[:4].tolist()}")
    tol = H.TOL[cfg.wdtype]
    orc = oracle.Oracle(mc, workloads.mtp_model_weights(_cpu(case.w_gpu), _cpu(mw)), cap_m)
    mw_cpu = _cpu(mw)
    final_norm = case.w_gpu["final_norm"].cpu().numpy()
    checked = agree = depths = 0
    kn, vn = sv.kv_from_library(mkl, mvl)
    for b in range(B):
        a = int(g["accepted"][b])
        c0 = int(case.ctx[b])
        rows = g["hidden"][cfg.n_layers - 1, b * K1:b * K1 + a + 1].astype(np.float64)
        bstate = np.stack([oracle.rmsnorm(r, final_norm, cfg.rms_eps) for r in rows])
        kc, vc = orc.kv_np(mk[b:b + 1], mv[b:b + 1])
        want, gaps = orc.mtp_draft(mw_cpu, kc, vc, 0, c0, a, drafts[b].numpy(),
                                   int(g["next_tok"][b]), bstate)
        sure = True
        for d in range(K):
            sure = sure and gaps[d] > tol
            depths += 1
            agree += int(got[b, d] == want[d])
            if sure:
                checked += 1
                assert got[b, d] == want[d], (
                    f"seq {b} depth {d + 1}: gpu {got[b, d]} oracle {want[d]} (gap {gaps[d]:.3g})")
        # the block's cache at the committed positions
        conv = (lambda t: t.float().cpu().numpy().astype(np.float64))
        for name, gt, ot in (("k", kn, kc), ("v", vn, vc)):
            gg = conv(gt[b, 0, :, c0:c0 + a + 1])
            oo = ot[0, 0, :, c0:c0 + a + 1]
            oo = oo.astype(np.float64) if cfg.kvdtype == "f32" else \
                (oo.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            rng = float(oo.max() - oo.min())
            assert float(np.abs(gg - oo).max()) <= tol * rng, f"seq {b}: block {name} cache"
    H.say(f"[{label}] drafts checked {checked}/{depths}, agree {agree}/{depths}")
    assert checked >= min_checked * depths
    dctx.close()
    run.close()


def test_draft_tiny_fp32(H):
    cfg = workloads.scaled(workloads.get_config("tiny_fp32"), batch=3, ctx=("uniform", 100, 200))
    _draft_case(H, cfg, "draft tiny_fp32", min_checked=0.9)


def test_draft_moe_b1(H):
    _draft_case(H, workloads.get_config("moe_b1"), "draft moe_b1", min_checked=0.0)


def test_draft_moe_batched_scaled(H):
    cfg = workloads.scaled(workloads.get_config("moe_b32"), n_layers=2, vocab=8192, batch=6,
                           ctx=("uniform", 50, 400))
    _draft_case(H, cfg, "draft moe scaled", min_checked=0.0)


def test_draft_dense_fp8_scaled(H):
    cfg = workloads.scaled(workloads.get_config("dense_fp8_b8"), n_layers=1, vocab=8192, batch=2,
                           k_draft=7, ctx=("uniform", 100, 300))
    _draft_case(H, cfg, "draft fp8 scaled", min_checked=0.0)


def test_draft_mxfp4_target(H):
    """The tied LM head in MXFP4 (a target with MXFP4 experts and LM head)."""
    _draft_case(H, workloads.get_config("moe_b1_mxfp4"), "draft moe_b1_mxfp4", min_checked=0.0)


def test_draft_failed_sequences_get_no_drafts(H):
    """A sequence whose verify step failed (accepted -1) or whose positions
    exceed the block cache gets drafts -1 and raises the error bits; the
    others are drafted normally."""
    import speculative_decoding_verify_step_amd as sv
    cfg = workloads.scaled(workloads.get_config("tiny_fp32"), batch=3, ctx=("fixed", 100))
    case = H.Case(cfg)
    run = H.GpuRun(case, batch=3)
    drafts = case.rtok[0][:3].clone()
    run.step(case.committed[:3], drafts, case.ctx[:3])
    mc = workloads.mtp_config(cfg)
    mw = workloads.mtp_weights(cfg, "cuda")
    cap_m = 192
    mk, mv = workloads.kv_cache(workloads.scaled(mc, batch=3), "cuda", capacity=cap_m)
    mkl, mvl = sv.kv_to_library(mk, mv)
    dctx = sv.DraftContext(mc, 3, cap_m, run.ctx.weights, mw)
    i32 = dict(dtype=torch.int32, device="cuda")
    acc = run.acc.clone()
    acc[1] = -1
    ctx_in = torch.tensor([100, 100, 190], **i32)       # sequence 2: 190 + (K+1) > 192
    out = torch.full((3, cfg.k_draft), -9, **i32)
    dctx.draft(mkl, mvl, run.ctx, ctx_in, acc, run.nxt, drafts.to(**i32).contiguous(), out)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[1] == -1) and np.all(o[2] == -1)
    assert np.all((o[0] >= 0) & (o[0] < cfg.vocab))
    # the capacity overflow is reported; the failed verify step was reported by its own context
    assert dctx.error_word(clear=True) == sv.SV_DEV_CAPACITY
    dctx.close()
    run.close()


def test_draft_verify_loop_replays_from_one_graph(H):
    """Three iterations of the device-resident loop (verify the drafts, then
    draft the next ones from the outcome; contexts and committed tokens carried
    on the device) captured into one HIP graph: each replay from the restored
    start state gives the eager loop's accepted lengths, tokens, contexts and
    drafts."""
    import speculative_decoding_verify_step_amd as sv
    cfg = workloads.scaled(workloads.get_config("moe_b32"), n_layers=2, vocab=8192, batch=4,
                           steps=4, ctx=("uniform", 100, 300))
    case = H.Case(cfg)
    B, S = cfg.batch, 3
    vc = sv.VerifyContext(cfg, B, case.cap, case.w_gpu)
    kc0, vc0 = sv.kv_to_library(case.k_nat[:B], case.v_nat[:B])
    mc = workloads.mtp_config(cfg)
    mw = workloads.mtp_weights(cfg, "cuda")
    mk0, mv0 = workloads.kv_cache(workloads.scaled(mc, batch=B), "cuda", capacity=case.cap)
    mk0, mv0 = sv.kv_to_library(mk0, mv0)
    dctx = sv.DraftContext(mc, B, case.cap, vc.weights, mw)
    kc, vcc, mk, mv = kc0.clone(), vc0.clone(), mk0.clone(), mv0.clone()
    i32 = dict(dtype=torch.int32, device="cuda")
    com0 = case.committed[:B].to(**i32)
    ctx0 = case.ctx[:B].to(**i32)
    d0 = case.rtok[0][:B].to(**i32).contiguous()
    coms = [torch.empty(B, **i32) for _ in range(S + 1)]
    ctxs = [torch.empty(B, **i32) for _ in range(S + 1)]
    drs = [torch.empty(B, cfg.k_draft, **i32) for _ in range(S + 1)]
    accs = [torch.empty(B, **i32) for _ in range(S)]

    def loop():
        for s_ in range(S):
            vc.step(kc, vcc, coms[s_], drs[s_], ctxs[s_], ctxs[s_ + 1], accs[s_], coms[s_ + 1])
            dctx.draft(mk, mv, vc, ctxs[s_], accs[s_], coms[s_ + 1], drs[s_], drs[s_ + 1])

    def restore():
        for t, t0 in ((kc, kc0), (vcc, vc0), (mk, mk0), (mv, mv0), (coms[0], com0),
                      (ctxs[0], ctx0), (drs[0], d0)):
            t.copy_(t0)

    outs = accs + coms + ctxs + drs
    restore()
    loop()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    assert vc.error_word() == 0 and dctx.error_word() == 0
    assert all(int(a.min()) >= 0 for a in accs)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        restore()
        loop()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        loop()
    for rep in range(3):
        restore()
        for t in accs + coms[1:] + ctxs[1:] + drs[1:]:
            t.fill_(-5)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, eager):
            assert torch.equal(got, want), f"replay {rep}"
    assert vc.error_word() == 0 and dctx.error_word() == 0
    dctx.close()
    vc.close()
