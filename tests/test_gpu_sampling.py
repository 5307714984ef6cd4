"""Sampled (rejection-sampling) verification on the GPU: parity with the CPU
oracle (oracle/sampling.py) and the lossless property checked directly.

Comparison rule.  The outcome of a sequence (accepted length, drawn token,
new context length) must be bit-identical to the oracle's whenever it is
certain under the arithmetic's error: every acceptance comparison keeps its
side and the final draw keeps its winner when every target probability may be
off by a relative DELTA and every Gumbel key by KEY_SLACK.  On the GPU's own
fp32 logits (the isolated sampling entry point, and the full step read back
through the debug logits) DELTA = KEY_SLACK = 1e-4 covers fp32 exp / log /
log-sum-exp rounding against the oracle's fp64; nearly every sequence is then
checked.  Against the oracle's own fp64 forward the logits themselves are
compared under the greedy tests' tolerance (2e-2 of each position's logit
range for bf16 weights, 1e-4 for fp32), and the outcome is checked where it is
certain under the logit error actually measured.
"""
import numpy as np
import pytest
import scipy.stats
import torch

import workloads

pytestmark = pytest.mark.gpu

DELTA = 1e-4
KEY_SLACK = 1e-4


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_harness
    return gpu_harness


@pytest.fixture(scope="module")
def S():
    from oracle import sampling
    return sampling


class SampleCtx:
    """A library context used only for the sampling entry point."""

    def __init__(self, cfg, max_batch):
        import speculative_decoding_verify_step_amd as sv
        self.sv = sv
        self.cfg = cfg
        self.handle = sv.spec_verify_init(sv.make_config(cfg, max_batch,
                                                         workloads.capacity_for(cfg)))

    def run(self, logits, drafts, q, u, tau, seed, offset, ctx_in):
        B = drafts.shape[0]
        dev = "cuda"
        lg = logits.to(dev, torch.float32).contiguous()
        dr = drafts.to(dev, torch.int32).contiguous()
        qq = q.to(dev, torch.float32).contiguous()
        uu = u.to(dev, torch.float32).contiguous()
        ci = ctx_in.to(dev, torch.int32).contiguous()
        co = torch.full((B,), -9, dtype=torch.int32, device=dev)
        acc = torch.full((B,), -9, dtype=torch.int32, device=dev)
        nxt = torch.full((B,), -9, dtype=torch.int32, device=dev)
        self.sv.spec_verify_sample_from_logits(self.handle, lg, dr, qq, uu, tau, seed, offset, ci,
                                               co, B, acc, nxt)
        torch.cuda.synchronize()
        return acc.cpu().numpy(), nxt.cpu().numpy(), co.cpu().numpy()

    def error_word(self, clear=True):
        return self.sv.spec_verify_error_word(self.handle, clear)

    def close(self):
        self.sv.spec_verify_destroy(self.handle)


def _logits(cfg, B, sigma, seed):
    g = torch.Generator().manual_seed(seed)
    return sigma * torch.randn(B, cfg.k_draft + 1, cfg.vocab, generator=g)


def _compare(S, H, label, logits, sd, tau, ga, gn, gc, ctx, B, min_checked=0.9):
    o = S.sampled_verify(logits.double().numpy(), sd["drafts"][:B].numpy(), sd["q"][:B].numpy(),
                         sd["u"][:B].numpy(), tau, sd["seed"], sd["offset"], delta=DELTA,
                         key_slack=KEY_SLACK)
    sure = o["accept_certain"] & o["draw_certain"]
    same = (ga == o["accepted"]) & (gn == o["next_tok"])
    H.say(f"[{label}] accepted gpu {ga[:8].tolist()} oracle {o['accepted'][:8].tolist()}; "
          f"certain {int(sure.sum())}/{B}, agree {int(same.sum())}/{B}, "
          f"kinds {sorted(set(o['kind']))}")
    for b in np.nonzero(sure)[0]:
        assert ga[b] == o["accepted"][b], f"seq {b}: accepted {ga[b]} vs {o['accepted'][b]}"
        assert gn[b] == o["next_tok"][b], f"seq {b}: token {gn[b]} vs {o['next_tok'][b]}"
        assert gc[b] == ctx[b] + o["accepted"][b] + 1
    assert sure.mean() >= min_checked, f"only {sure.mean():.2f} of the sequences are certain"
    return o


@pytest.mark.parametrize("name,B,tau,sigma", [
    ("tiny_fp32", 8, 1.0, 0.3),          # V = 1024: one partial vocabulary tile
    ("moe_b1", 64, 1.0, 0.716),          # V = 129,280 at the batch-64 shape
    ("moe_b1", 16, 0.6, 2.0),            # sharper target, temperature below 1
    ("dense_fp8_b8", 8, 1.3, 1.0),       # V = 151,936, K = 31
])
def test_sample_from_logits_matches_oracle(H, S, name, B, tau, sigma):
    cfg = workloads.scaled(workloads.get_config(name), batch=B)
    H.say(f"[sample {name}] B={B} V={cfg.vocab} K={cfg.k_draft} tau={tau} sigma={sigma}")
    sd = workloads.sampled_drafts(cfg)
    logits = _logits(cfg, B, sigma, 101)
    ctx = torch.arange(B, dtype=torch.int32) + 10
    sc = SampleCtx(cfg, B)
    ga, gn, gc = sc.run(logits, sd["drafts"], sd["q"], sd["u"], tau, sd["seed"], sd["offset"], ctx)
    assert sc.error_word() == 0
    assert np.all((ga >= 0) & (ga <= cfg.k_draft)) and np.all((gn >= 0) & (gn < cfg.vocab))
    _compare(S, H, f"sample {name}", logits, sd, tau, ga, gn, gc, ctx.numpy(), B)
    # same inputs, same outcome (every reduction has a fixed order)
    ga2, gn2, gc2 = sc.run(logits, sd["drafts"], sd["q"], sd["u"], tau, sd["seed"], sd["offset"], ctx)
    assert np.array_equal(ga, ga2) and np.array_equal(gn, gn2) and np.array_equal(gc, gc2)
    sc.close()


def test_sample_from_logits_residual_and_bonus_paths(H, S):
    """Drafts the target cannot produce (q one-hot where p is tiny) are always
    rejected and replaced from the residual; drafts drawn from q = p are
    always kept and end with the bonus draw."""
    cfg = workloads.scaled(workloads.get_config("tiny_fp32"), batch=32)
    B, K, V = 32, cfg.k_draft, cfg.vocab
    logits = _logits(cfg, B, 1.0, 7)
    logits[:16, :, 5] = -30.0                      # p(5) ~ 1e-13 on the first half
    q = torch.zeros(B, K, V)
    drafts = torch.zeros(B, K, dtype=torch.int32)
    q[:16, :, 5] = 1.0
    drafts[:16] = 5
    p = torch.softmax(logits[16:, :K].double(), -1)
    q[16:] = p.float()
    g = torch.Generator().manual_seed(3)
    drafts[16:] = torch.multinomial(p.reshape(-1, V), 1, generator=g).reshape(16, K).to(torch.int32)
    u = torch.rand(B, K, generator=g)
    sd = {"drafts": drafts, "q": q, "u": u, "seed": 1234567, "offset": 9}
    ctx = torch.zeros(B, dtype=torch.int32)
    sc = SampleCtx(cfg, B)
    ga, gn, gc = sc.run(logits, drafts, q, u, 1.0, sd["seed"], sd["offset"], ctx)
    assert np.all(ga[:16] == 0) and np.all(gn[:16] != 5)
    o = _compare(S, H, "paths", logits, sd, 1.0, ga, gn, gc, ctx.numpy(), B)
    assert set(o["kind"][:16]) == {"residual"}
    sc.close()


def test_first_token_follows_the_target_on_gpu(H):
    """The lossless property measured on the GPU alone: over 8,192 sequences
    sharing p_0 and q_1 (independent noise per sequence), the first token a
    step emits follows p_0 (chi-square), and drafts are kept at the rate
    sum_v min(p_0(v), q_1(v))."""
    base = workloads.get_config("tiny_fp32")
    cfg = workloads.scaled(base, ffn="dense", dense_inter=128, n_experts=0, top_k=0,
                           n_shared=0, vocab=64, k_draft=1, batch=8192)
    B, V = cfg.batch, cfg.vocab
    g = torch.Generator().manual_seed(21)
    L0 = 1.5 * torch.randn(V, generator=g, dtype=torch.float64)
    tau = 0.9
    p0 = torch.softmax(L0 / tau, 0)
    q1 = torch.softmax(1.5 * torch.randn(V, generator=g, dtype=torch.float64), 0)
    logits = torch.zeros(B, 2, V)
    logits[:, 0] = L0.float()
    drafts = torch.multinomial(q1, B, replacement=True, generator=g).to(torch.int32).reshape(B, 1)
    u = torch.rand(B, 1, generator=g)
    q = q1.float().reshape(1, 1, V).expand(B, 1, V).contiguous()
    sc = SampleCtx(cfg, B)
    ga, gn, _ = sc.run(logits, drafts, q, u, tau, 0xDEADBEEF12345, 77, torch.zeros(B, dtype=torch.int32))
    first = np.where(ga == 1, drafts[:, 0].numpy(), gn)
    counts = np.bincount(first, minlength=V).astype(np.float64)
    exp = p0.numpy() * B
    big = exp >= 5                                  # pool the rare entries into one cell
    obs = np.append(counts[big], counts[~big].sum())
    ex = np.append(exp[big], exp[~big].sum())
    pval = scipy.stats.chisquare(obs, ex).pvalue
    acc = float(torch.minimum(p0, q1).sum())
    rate = float((ga == 1).mean())
    H.say(f"[lossless] chi-square p = {pval:.3g}; keep rate {rate:.4f} vs {acc:.4f}")
    assert pval > 1e-3
    assert abs(rate - acc) < 4 * np.sqrt(acc * (1 - acc) / B)
    sc.close()


def test_sample_errors_and_noise_streams(H):
    cfg = workloads.scaled(workloads.get_config("tiny_fp32"), batch=6)
    B = 6
    sd = workloads.sampled_drafts(cfg)
    logits = _logits(cfg, B, 1.0, 5)
    logits[2, 1, 77] = float("nan")                  # a NaN logit in sequence 2
    drafts = sd["drafts"].clone()
    drafts[4, 0] = cfg.vocab                         # an out-of-range draft in sequence 4
    ctx = torch.full((B,), 40, dtype=torch.int32)
    sc = SampleCtx(cfg, B)
    ga, gn, gc = sc.run(logits, drafts, sd["q"], sd["u"], 1.0, sd["seed"], 0, ctx)
    assert ga[2] == -1 and gn[2] == -1 and gc[2] == 40
    assert ga[4] == -1 and gn[4] == -1 and gc[4] == 40
    ok = [0, 1, 3, 5]
    assert np.all(ga[ok] >= 0) and np.all(gc[ok] == 40 + ga[ok] + 1)
    import speculative_decoding_verify_step_amd as sv
    assert sc.error_word() == sv.SV_DEV_NAN_LOGIT | sv.SV_DEV_BAD_TOKEN
    # another offset draws other tokens (independent noise)
    clean = _logits(cfg, B, 1.0, 5)
    outs = [sc.run(clean, sd["drafts"], sd["q"], sd["u"], 1.0, sd["seed"], off, ctx)[1]
            for off in range(4)]
    assert len({tuple(o.tolist()) for o in outs}) > 1
    with pytest.raises(sv.SpecVerifyError):
        sc.run(clean, sd["drafts"], sd["q"], sd["u"], 0.0, sd["seed"], 0, ctx)
    with pytest.raises(sv.SpecVerifyError):
        sc.run(clean, sd["drafts"], sd["q"], sd["u"], float("inf"), sd["seed"], 0, ctx)
    sc.close()


@pytest.mark.parametrize("name,overrides", [
    ("tiny_fp32", {}),
    ("moe_b1", {}),
    ("moe_b32", {"n_layers": 2, "batch": 6, "ctx": ("uniform", 300, 700)}),
    ("dense_fp8_b8", {"n_layers": 1, "batch": 2, "ctx": ("uniform", 200, 600), "k_draft": 7}),
])
def test_sampled_step_matches_oracle(H, S, name, overrides):
    """The whole sampled step: logits against the oracle's forward, the
    outcome against the oracle's sampling on the GPU's logits (certain set,
    nearly every sequence) and on the oracle's own logits (certain under the
    measured logit error), the new cache entries against the oracle's."""
    cfg = workloads.scaled(workloads.get_config(name), **overrides) if overrides else \
        workloads.get_config(name)
    case = H.Case(cfg)
    B = cfg.batch
    sd = workloads.sampled_drafts(cfg)
    tau = 0.8
    H.say(f"[sampled step {cfg.name}] B={B} L={cfg.n_layers} V={cfg.vocab} K={cfg.k_draft} "
          f"ctx={case.ctx[:B].tolist()[:8]}")
    run = H.GpuRun(case, batch=B)
    dev = "cuda"
    com = case.committed[:B].to(dev, torch.int32).contiguous()
    dr = sd["drafts"].to(dev).contiguous()
    ci = case.ctx[:B].to(dev, torch.int32).contiguous()
    run.ctx.step_sampled(run.kc, run.vc, com, dr, sd["q"].to(dev).contiguous(),
                         sd["u"].to(dev).contiguous(), tau, sd["seed"], sd["offset"], ci,
                         run.ctx_out, run.acc, run.nxt, batch=B)
    torch.cuda.synchronize()
    ga, gn, gc = run.acc.cpu().numpy(), run.nxt.cpu().numpy(), run.ctx_out.cpu().numpy()
    glog = run.logits.cpu()
    assert run.ctx.error_word(clear=True) == 0
    H.say(f"[sampled step {cfg.name}] gpu accepted {ga[:8].tolist()} next {gn[:8].tolist()}")
    _compare(S, H, f"sampled step {cfg.name} / gpu logits", glog, sd, tau, ga, gn, gc,
             case.ctx[:B].numpy(), B)
    orc = case.oracle()
    tol = H.TOL[cfg.wdtype]
    stats = {}
    o_logits = np.zeros((B, cfg.k_draft + 1, cfg.vocab))
    for b in range(B):
        kc, vc = case.oracle_kv(b)
        forced = rlg = None
        if cfg.ffn == "moe":
            K1 = cfg.k_draft + 1
            forced = run.routing.cpu().numpy()[:, b * K1:(b + 1) * K1][None]
            rlg = run.rlogits.cpu().numpy()[:, b * K1:(b + 1) * K1]
        o = orc.verify_step(kc, vc, [int(case.committed[b])], sd["drafts"][b:b + 1].numpy(),
                            [int(case.ctx[b])], want_logits=True, force_sel=forced,
                            want_routing=forced is not None)
        H.check_routing(cfg, forced, o, stats, label=f"seq {b}", rl_gpu=rlg)
        o_logits[b] = o["logits"][0]
        for j in range(cfg.k_draft + 1):
            lo, lg = o["logits"][0, j], glog[b, j].double().numpy()
            rng = float(lo.max() - lo.min())
            assert float(np.abs(lg - lo).max()) <= tol * rng, f"seq {b} pos {j}: logits"
        H.compare_new_kv(cfg, run, b, kc, vc, int(case.ctx[b]), stats)
    err = float(np.abs(glog.double().numpy() - o_logits).max())
    delta = float(np.expm1(2 * err / tau)) + DELTA
    o = S.sampled_verify(o_logits, sd["drafts"].numpy(), sd["q"].numpy(), sd["u"].numpy(), tau,
                         sd["seed"], sd["offset"], delta=delta, key_slack=2 * err / tau + KEY_SLACK)
    sure = o["accept_certain"] & o["draw_certain"]
    for b in np.nonzero(sure)[0]:
        assert ga[b] == o["accepted"][b] and gn[b] == o["next_tok"][b]
    if cfg.ffn == "moe":
        H.assert_forced_cap(stats, f"sampled step {cfg.name}")
    H.say(f"[sampled step {cfg.name}] oracle-forward check: max logit err {err:.2e}, "
          f"certain {int(sure.sum())}/{B}, agree {int(((ga == o['accepted']) & (gn == o['next_tok'])).sum())}/{B}")
    run.close()
