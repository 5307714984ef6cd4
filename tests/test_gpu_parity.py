"""Parity of the HIP verify step with the CPU oracle on seeded inputs.

Every test calls the library through its C ABI (the ctypes binding) and
compares with the oracle under the rules in gpu_harness.  Sizes: the tiny and
batch-1 workloads at full size; scaled versions of the batched MoE, the fp8
dense GQA and the chained long-context workloads that span several tiles,
chunks and a ragged tail and that the oracle finishes in seconds.
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


def _poison_dead_slots(case, B):
    """Positions at or past ctx + K + 1 (never written by the step, never read
    by any query) filled with NaN, +Inf and -Inf in turn."""
    K1 = case.cfg.k_draft + 1
    pat = torch.tensor([float("nan"), float("inf"), float("-inf")])
    for b in range(B):
        c = int(case.ctx[b]) + K1
        n = case.cap - c
        fill = pat.repeat(n // 3 + 1)[:n].to(case.k_nat.dtype).to(case.k_nat.device)
        case.k_nat[b, :, :, c:] = fill[:, None]
        case.v_nat[b, :, :, c:] = fill.flip(0)[:, None]


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _verify_case(H, cfg, sampled=None, batch=None, check_kv=True, label="", poison=False,
                 layout="tiled16"):
    case = H.Case(cfg)
    B = cfg.batch if batch is None else batch
    if poison:
        _poison_dead_slots(case, B)
    sampled = list(range(B)) if sampled is None else sampled
    H.say(f"[{label}] {cfg.name}: B={B} L={cfg.n_layers} H={cfg.hidden} V={cfg.vocab} "
          f"K={cfg.k_draft} cap={case.cap} ctx={case.ctx[:B].tolist()[:8]} sampled={sampled}")
    drafts = case.drafts(sampled)
    run = H.GpuRun(case, batch=B, layout=layout)
    g = run.step(case.committed[:B], drafts[:B], case.ctx[:B])
    H.say(f"[{label}] gpu step done: accepted={g['accepted'][:8].tolist()}")
    orc = case.oracle()
    stats = {}
    for b in sampled:
        kc, vc = case.oracle_kv(b)
        forced = run.routing_of(g, b)
        o = orc.verify_step(kc, vc, [int(case.committed[b])], drafts[b:b + 1].numpy(),
                            [int(case.ctx[b])], want_logits=True, want_layer_hidden=True,
                            force_sel=forced, want_routing=forced is not None)
        H.check_routing(cfg, forced, o, stats, label=f"seq {b}", rl_gpu=run.rlogits_of(g, b))
        H.compare_sequence(cfg, g, b, o, 0, stats)
        if check_kv:
            H.compare_new_kv(cfg, run, b, kc, vc, int(case.ctx[b]), stats)
    # the step wrote nothing outside the K+1 new slots of each sequence
    K1 = cfg.k_draft + 1
    import speculative_decoding_verify_step_amd as sv
    k_after, v_after = sv.kv_from_library(run.kc, run.vc)
    for b in range(B):
        c = int(case.ctx[b])
        for before, after, name in ((case.k_nat[b].clone(), k_after[b].clone(), "K"),
                                    (case.v_nat[b].clone(), v_after[b].clone(), "V")):
            before[:, :, c:c + K1] = 0
            after[:, :, c:c + K1] = 0
            assert torch.equal(_bits(before), _bits(after)), \
                f"seq {b}: {name} cache changed outside the new slots"
    H.say(f"[{label}] stats {stats}")
    if cfg.ffn == "moe":
        H.assert_forced_cap(stats, label)
    run.close()
    return stats, g


def test_tiny_fp32_full_size(H):
    cfg = workloads.get_config("tiny_fp32")
    stats, _ = _verify_case(H, cfg, label="tiny_fp32")
    assert stats["max_rel_logit_err"] < 1e-4
    assert stats["accept_checked"] == 1


@pytest.mark.parametrize("batch,k_draft,n_q,n_kv,head_dim", [(3, 7, 8, 2, 64), (17, 3, 4, 4, 64),
                                                            (5, 3, 2, 2, 128), (9, 3, 4, 2, 128)])
def test_fp32_more_rows(H, batch, k_draft, n_q, n_kv, head_dim):
    """The fp32 path beyond the tiny workload's four rows: grouped-query heads
    (4 per KV head, K = 7: 32 rows per KV head, two fragments per wave of the
    split-KV kernel) with contexts up to 1,500 (the merge over up to 24
    chunks), 68 rows (the large-row GEMMs and the separate embedding and
    rotary kernels at fp32), and head dimension 128 at 20 and 36 rows (the
    fused QKV kernel with two and four row fragments)."""
    cfg = workloads.scaled(workloads.get_config("tiny_fp32"), batch=batch, k_draft=k_draft, n_q=n_q,
                           n_kv=n_kv, head_dim=head_dim, ctx=("uniform", 60, 1500))
    stats, _ = _verify_case(H, cfg, label=f"fp32_b{batch}_k{k_draft}_d{head_dim}")
    assert stats["max_rel_logit_err"] < 1e-4


def test_moe_batch1_full_size(H):
    cfg = workloads.get_config("moe_b1")
    stats, _ = _verify_case(H, cfg, label="moe_b1")
    assert stats["accept_agree"] == 1


def test_moe_batched_scaled(H):
    """The batched MoE stack with fewer layers and a smaller vocabulary; the
    context range spans several attention chunks and a ragged last tile."""
    cfg = workloads.scaled(workloads.get_config("moe_b32"), n_layers=3, vocab=8192, batch=20,
                           ctx=("uniform", 30, 700))
    stats, _ = _verify_case(H, cfg, label="moe_b32_scaled")   # 80 rows: large-row GEMM path
    assert stats["argmax_agree"] >= 0.9 * stats["positions"]


@pytest.mark.parametrize("batch,n_experts,top_k", [(5, 16, 4), (20, 16, 4), (16, 8, 6), (10, 4, 2),
                                                  (14, 4, 3)])
def test_moe_small_shapes(H, batch, n_experts, top_k):
    """Small MoE shapes: head_dim 128 with 2 heads, one shared expert, contexts
    from 1 token, norm gains away from 1.  Rows per expert ~1 (one-wave expert
    tiles), ~20 (32-row tiles of the large-row kernel) and ~48 (64-row tiles),
    and on the few-row kernel (under 64 rows) ~20 and ~42 (32- and 64-row
    expert tiles)."""
    cfg = workloads.scaled(workloads.get_config("moe_b1"), n_layers=2, hidden=256, n_q=2, n_kv=2,
                           n_experts=n_experts, expert_inter=128, top_k=top_k, n_shared=1,
                           vocab=2048, batch=batch, ctx=("uniform", 1, 200), norm_gain_std=0.2)
    _verify_case(H, cfg, label=f"moe_small_shapes_b{batch}_e{n_experts}_k{top_k}")


@pytest.mark.parametrize("batch,n_experts,top_k,n_shared", [(4, 32, 4, 2), (1, 64, 8, 0), (4, 16, 2, 3),
                                                            (2, 8, 2, 8)])
def test_moe_few_assignments(H, batch, n_experts, top_k, n_shared):
    """Few assignments (T <= 16, T * top_k <= 64, at most 64 experts): the
    grouped GEMMs and the combine take expert tiles and slots from the
    selections.  Covers all 64 lanes holding an assignment (16 rows x top-4),
    none, two, three and eight shared experts (the combine's shared-expert
    loads sized for 1, 2, 4 and 8)."""
    cfg = workloads.scaled(workloads.get_config("moe_b1"), n_layers=2, hidden=256, n_q=2, n_kv=2,
                           n_experts=n_experts, expert_inter=128, top_k=top_k, n_shared=n_shared,
                           vocab=2048, batch=batch, ctx=("uniform", 1, 200), norm_gain_std=0.2)
    _verify_case(H, cfg, label=f"moe_few_b{batch}_e{n_experts}_k{top_k}_s{n_shared}")


@pytest.mark.parametrize("batch,n_experts,top_k", [(3, 16, 4), (20, 16, 4)])
def test_moe_fp8_experts(H, batch, n_experts, top_k):
    """e4m3 weights with per-row scales in the MoE decoder (router, experts,
    projections, LM head): 12 rows (the few-row kernels, tiles and slots
    implied by the selections) and 80 rows (the grouped large-row kernel
    with device-built tiles)."""
    cfg = workloads.scaled(workloads.get_config("moe_b1"), n_layers=2, hidden=256, n_q=2, n_kv=2,
                           n_experts=n_experts, expert_inter=128, top_k=top_k, n_shared=1,
                           vocab=2048, batch=batch, ctx=("uniform", 1, 200), norm_gain_std=0.2,
                           wdtype="fp8")
    _verify_case(H, cfg, label=f"moe_fp8_b{batch}_e{n_experts}_k{top_k}")


def test_moe_fp8_batch1_shapes(H):
    """The batch-1 MoE layer's shapes (hidden 1,280, 64 experts, top-6, two
    shared experts, expert width 896) with e4m3 weights: the selections made
    inside the expert gate/up kernel, the K-split expert down projection and
    the small-row LM head, on fp8 operands (smaller vocabulary)."""
    cfg = workloads.scaled(workloads.get_config("moe_b1"), vocab=8192, wdtype="fp8")
    stats, _ = _verify_case(H, cfg, label="moe_fp8_b1")
    assert stats["argmax_agree"] >= 0.75 * stats["positions"]


def test_dense_fp8_gqa_scaled(H):
    """Block drafts (K = 31) on the dense GQA decoder with e4m3 weights:
    4 query heads per KV head, 128 query rows per KV head."""
    cfg = workloads.scaled(workloads.get_config("dense_fp8_b8"), n_layers=2, hidden=512, n_q=8,
                           n_kv=2, dense_inter=1024, vocab=4096, batch=3,
                           ctx=("uniform", 100, 900))
    stats, _ = _verify_case(H, cfg, label="dense_fp8_scaled")
    assert stats["argmax_agree"] >= 0.8 * stats["positions"]


@pytest.mark.parametrize("k_draft,head_dim,waves", [(15, 128, 2), (63, 128, 8), (31, 64, 4), (7, 64, 1),
                                                    (4, 128, 1), (15, 64, 2), (63, 64, 8)])
def test_gqa_many_rows_attention_shapes(H, k_draft, head_dim, waves):
    """The LDS-ring attention kernel (17 .. 256 query rows per KV head) at
    each of its workgroup shapes: (K+1) x 4 grouped query heads = 64, 256,
    128 and 32 rows (2, 8, 4 and 1 waves of two 16-row fragments), head
    dimension 128 and 64, contexts that end mid-tile and mid-chunk; and 20
    rows, whose second fragment holds 12 padding rows (never written, and
    the tiles before the context end skip the mask for every row)."""
    cfg = workloads.scaled(workloads.get_config("dense_fp8_b8"), n_layers=1, hidden=512, n_q=8,
                           n_kv=2, head_dim=head_dim, dense_inter=1024, vocab=4096, batch=2,
                           k_draft=k_draft, ctx=("uniform", 60, 700))
    rows = (k_draft + 1) * (cfg.n_q // cfg.n_kv)
    nw = 1                                   # the library's rule: 2 nw fragments >= ceil(rows / 16)
    while 2 * nw < -(-rows // 16):
        nw *= 2
    assert 17 <= rows <= 256 and nw == waves
    stats, _ = _verify_case(H, cfg, label=f"gqa_rows{rows}_d{head_dim}")
    assert stats["argmax_agree"] >= 0.8 * stats["positions"]


@pytest.mark.parametrize("batch,k_draft", [(1, 31), (3, 15)])
def test_dense_fp8_few_rows(H, batch, k_draft):
    """fp8 weights at 32 and 48 rows: the fused embedding + QKV + rotary
    kernel and the few-row GEMMs with two and four row fragments."""
    cfg = workloads.scaled(workloads.get_config("dense_fp8_b8"), n_layers=2, hidden=512, n_q=8,
                           n_kv=2, dense_inter=1024, vocab=4096, batch=batch, k_draft=k_draft,
                           ctx=("uniform", 60, 500))
    stats, _ = _verify_case(H, cfg, label=f"fp8_rows{batch * (k_draft + 1)}")
    assert stats["argmax_agree"] >= 0.8 * stats["positions"]


def test_gqa_more_than_256_rows_per_kv_head(H):
    """512 query rows per KV head (K = 63, 8 query heads per KV head), past
    the LDS-ring kernel's 256: the split-KV kernel with four fragments per
    wave and eight query groups per KV head."""
    cfg = workloads.scaled(workloads.get_config("dense_fp8_b8"), n_layers=1, hidden=512, n_q=16,
                           n_kv=2, dense_inter=1024, vocab=4096, batch=1, k_draft=63,
                           ctx=("uniform", 100, 700))
    assert (cfg.k_draft + 1) * (cfg.n_q // cfg.n_kv) == 512
    stats, _ = _verify_case(H, cfg, label="gqa_rows512")
    assert stats["argmax_agree"] >= 0.8 * stats["positions"]


def test_gqa_split_kernel_one_fragment(H):
    """Grouped-query attention on the split-KV kernel: K = 3 with 4 query
    heads per KV head gives 16 rows per KV head (one fragment, below the
    LDS-ring kernel's 17), so each fragment mixes the rows of 4 query heads
    at 4 positions and the causal limit differs from row to row."""
    cfg = workloads.scaled(workloads.get_config("dense_fp8_b8"), n_layers=2, hidden=512, n_q=8,
                           n_kv=2, dense_inter=1024, vocab=4096, batch=6, k_draft=3,
                           ctx=("uniform", 30, 700))
    assert (cfg.k_draft + 1) * (cfg.n_q // cfg.n_kv) == 16
    stats, _ = _verify_case(H, cfg, label="gqa_split_16rows")
    assert stats["argmax_agree"] >= 0.8 * stats["positions"]


@pytest.mark.parametrize("batch", [3, 5, 9])
def test_dense_bf16_ffn_row_counts(H, batch):
    """A dense SwiGLU decoder with bf16 weights (the dense workload's shape in
    bf16, scaled) at 96, 160 and 288 rows (K = 31): the bf16 dense path's
    large-row kernels -- 128-row SwiGLU tiles up to 128 rows, the 32x32
    SwiGLU and projection kernel above 128, the LDS-staged LM head up to 256
    rows and the 32x32 argmax LM head above 256."""
    cfg = workloads.scaled(workloads.get_config("dense_fp8_b8"), n_layers=2, hidden=512, n_q=8,
                           n_kv=2, dense_inter=1024, vocab=4096, batch=batch, wdtype="bf16",
                           ctx=("uniform", 60, 500))
    stats, _ = _verify_case(H, cfg, label=f"dense_bf16_b{batch}")
    assert stats["argmax_agree"] >= 0.8 * stats["positions"]


@pytest.mark.parametrize("ctx", [3000, 9000])
def test_long_context_batch1_chunk_merge(H, ctx):
    """Batch 1 with a 3,000- or 9,000-position context: 64-key attention
    chunks, so the merge combines about 47 or 140 chunk partials per row (two
    or eight chunk weights per lane)."""
    cfg = workloads.scaled(workloads.get_config("moe_b1"), vocab=8192, ctx=("fixed", ctx))
    _verify_case(H, cfg, label=f"b1_ctx{ctx}")


@pytest.mark.parametrize("ctx", [3000, 9000])
def test_long_context_fp32_chunk_merge(H, ctx):
    """The fp32 path at a 3,000- or 9,000-position context: the split-KV
    kernel's 64-key chunks and the fp32 merge over about 47 or 141 chunk
    partials per row (two or eight chunk weights per lane)."""
    cfg = workloads.scaled(workloads.get_config("tiny_fp32"), ctx=("fixed", ctx))
    stats, _ = _verify_case(H, cfg, label=f"fp32_ctx{ctx}")
    assert stats["max_rel_logit_err"] < 1e-4


def test_mha_head_dim_64(H):
    """Multi-head attention with head dimension 64 (20 heads of 64 over
    hidden 1,280) on the split-KV kernel."""
    cfg = workloads.scaled(workloads.get_config("moe_b32"), n_layers=2, n_q=20, n_kv=20, head_dim=64,
                           vocab=4096, batch=3, ctx=("uniform", 50, 600))
    _verify_case(H, cfg, label="mha_d64")


@pytest.mark.parametrize("batch", [24, 40])
def test_lds_lm_head_ragged_vocabulary(H, batch):
    """The LDS-staged bf16 LM head on both of its tile shapes -- 96 rows on
    128 x 512 tiles, 160 rows on 256 x 256 tiles -- with a vocabulary that
    ends inside the last tile (5,008 = 9 x 512 + 400 = 19 x 256 + 144; the
    library takes vocabularies in multiples of 16): the
    argmax over the partial tile and the tile keys the acceptance reads."""
    cfg = workloads.scaled(workloads.get_config("moe_b32"), n_layers=1, vocab=5008, batch=batch,
                           ctx=("uniform", 30, 400))
    stats, g = _verify_case(H, cfg, sampled=[0, batch // 2, batch - 1], label=f"lm_head_lds_b{batch}")
    assert np.all(g["target"] >= 0) and np.all(g["target"] < cfg.vocab)
    assert stats["argmax_agree"] >= 0.8 * stats["positions"]


def test_dense_fp8_gqa_full_width_sampled(H):
    """The full fp8 dense layer width (hidden 2560, 32/8 heads, I 9728, vocab
    151,936) with 2 layers; two sequences of the batch checked."""
    cfg = workloads.scaled(workloads.get_config("dense_fp8_b8"), n_layers=2)
    _verify_case(H, cfg, sampled=[5], label="dense_fp8_wide")


def test_fp8_lds_projections_ragged(H):
    """fp8 projections on the LDS-staged kernel (K splits of 16 or more
    64-long steps) with ragged tiles: 160 rows (row tiles of 64, 64, 32) and
    hidden 1,216 = 4 x 256 + 192 output columns.  The O projection (K =
    16 x 128 = 2,048) and the down projection (K = 2,048) each run 2 splits of
    16 steps there; QKV and gate/up (K = 1,216, not a multiple of the 128-long
    chunk) take the small-row kernel."""
    cfg = workloads.scaled(workloads.get_config("dense_fp8_b8"), n_layers=2, hidden=1216, n_q=16,
                           n_kv=4, dense_inter=2048, vocab=4096, batch=5,
                           ctx=("uniform", 100, 900))
    stats, _ = _verify_case(H, cfg, label="fp8_lds_ragged")
    assert stats["argmax_agree"] >= 0.8 * stats["positions"]


@pytest.mark.parametrize("name,overrides", [
    ("tiny_fp32", {"batch": 3, "ctx": ("uniform", 20, 400)}),
    ("moe_b32", {"n_layers": 2, "vocab": 4096, "batch": 5, "ctx": ("uniform", 30, 500)}),
    ("dense_fp8_b8", {"n_layers": 1, "hidden": 512, "n_q": 8, "n_kv": 2, "dense_inter": 1024,
                      "vocab": 4096, "batch": 2, "k_draft": 7, "ctx": ("uniform", 50, 300)}),
])
def test_dead_cache_slots_may_hold_nan_and_inf(H, name, overrides):
    """Cache slots past the newest position of a sequence are dead (never
    written by the step, masked for every query) and may hold any bit
    pattern: filled with NaN / +-Inf, the step still matches the oracle and
    raises no error."""
    cfg = workloads.scaled(workloads.get_config(name), **overrides)
    stats, g = _verify_case(H, cfg, label=f"dead_slots_{name}", poison=True)
    assert np.all(g["accepted"] >= 0)
    assert np.all(np.isfinite(g["logits"]))


def test_deterministic_reruns(H):
    cfg = workloads.scaled(workloads.get_config("moe_b32"), n_layers=2, vocab=4096, batch=6,
                           ctx=("uniform", 50, 400))
    case = H.Case(cfg)
    H.say("[determinism] two identical steps")
    outs = []
    for _ in range(2):
        run = H.GpuRun(case)
        outs.append(run.step(case.committed, case.rtok[0], case.ctx))
        run.close()
    for k in ("logits", "hidden", "target", "accepted", "next_tok", "ctx_out"):
        assert np.array_equal(outs[0][k], outs[1][k], equal_nan=True), k


def test_chained_steps_scaled(H):
    """Verify steps chained on the device: ctx_lens_out aliases ctx_lens_in,
    next_tok becomes the next committed token, and the cache keeps the K/V of
    accepted positions (rollback by length).  The oracle runs the same chain
    on its own caches; every step is compared."""
    cfg = workloads.scaled(workloads.get_config("moe_b64_long"), n_layers=2, vocab=4096,
                           batch=8, steps=12, ctx=("loguniform", 20, 600))
    case = H.Case(cfg)
    B, K = cfg.batch, cfg.k_draft
    run = H.GpuRun(case)
    orc = case.oracle()
    kv = {b: case.oracle_kv(b) for b in range(B)}
    ctx_dev = case.ctx.to("cuda", torch.int32).clone()
    com = case.committed.clone()
    ctx_cpu = case.ctx.clone()
    stats = {}
    for s in range(cfg.steps):
        H.say(f"[chained] step {s} ctx={ctx_cpu.tolist()}")
        drafts = case.drafts(range(B), step=s, committed=com, ctx=ctx_cpu, kv=kv)
        g = run.step(com, drafts, ctx_dev, ctx_out=ctx_dev)
        for b in range(B):
            kc, vc = kv[b]
            forced = run.routing_of(g, b)
            o = orc.verify_step(kc, vc, [int(com[b])], drafts[b:b + 1].numpy(),
                                [int(ctx_cpu[b])], want_logits=True, force_sel=forced,
                                want_routing=True)
            H.check_routing(cfg, forced, o, stats, label=f"step {s} seq {b}",
                            rl_gpu=run.rlogits_of(g, b))
            H.compare_sequence(cfg, g, b, o, 0, stats, check_hidden=False)
            # continue both chains from the oracle's decision
            com[b] = int(o["next_tok"][0])
            ctx_cpu[b] = int(o["ctx_out"][0])
        ctx_dev.copy_(ctx_cpu.to("cuda", torch.int32))
    H.say(f"[chained] stats {stats}")
    H.assert_forced_cap(stats, "chained")
    assert stats["accept_agree"] >= 0.9 * stats["sequences"]
    assert int(ctx_cpu.min()) > int(case.ctx.min())
    run.close()


def test_accept_from_identical_logits_bit_exact(H):
    """Acceptance and commit fed the same fp32 logits as the oracle's rule:
    exact, including ties (lowest index wins) and a NaN position."""
    import oracle
    cfg = workloads.scaled(workloads.get_config("tiny_fp32"), batch=7, vocab=50000)
    case_cap = 4096
    import speculative_decoding_verify_step_amd as sv
    B, K, V = cfg.batch, cfg.k_draft, cfg.vocab
    w = workloads.make_weights(cfg, "cuda")
    ctx = sv.VerifyContext(cfg, B, case_cap, w)
    rng = np.random.default_rng(11)
    logits = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    g = logits.argmax(-1)
    # plant ties: a second index with the same maximum value (lower index must win)
    for b in range(B):
        for j in range(K + 1):
            top = g[b, j]
            other = (top + 1 + b * 7 + j) % V
            logits[b, j, other] = logits[b, j, top]
    drafts = np.zeros((B, K), np.int32)
    want_g = np.array([[oracle.argmax(logits[b, j].astype(np.float64)) for j in range(K + 1)]
                       for b in range(B)])
    # sequence b accepts min(b, K) drafts, then a wrong one
    for b in range(B):
        for i in range(K):
            drafts[b, i] = want_g[b, i] if i < min(b, K) else (want_g[b, i] + 1) % V
    logits[6, 2, 123] = np.nan
    ctx_in = torch.tensor([100 + b for b in range(B)], dtype=torch.int32, device="cuda")
    ctx_out = torch.zeros_like(ctx_in)
    acc = torch.zeros_like(ctx_in)
    nxt = torch.zeros_like(ctx_in)
    tgt = torch.zeros((B, K + 1), dtype=torch.int32, device="cuda")
    H.say("[accept_from_logits] B=7 V=50000 with planted ties and one NaN")
    ctx.accept_from_logits(torch.from_numpy(logits).cuda(), torch.from_numpy(drafts).cuda(), ctx_in,
                           ctx_out, acc, nxt, tgt)
    torch.cuda.synchronize()
    assert ctx.error_word(clear=True) & sv.SV_DEV_NAN_LOGIT
    for b in range(B):
        if b == 6:
            assert acc[b].item() == -1 and nxt[b].item() == -1 and ctx_out[b].item() == 100 + b
            continue
        a, n = oracle.accept(want_g[b], drafts[b])
        assert np.array_equal(tgt[b].cpu().numpy(), want_g[b])
        assert (acc[b].item(), nxt[b].item(), ctx_out[b].item()) == (a, n, 100 + b + a + 1)
    ctx.close()


def test_device_side_errors_are_reported_without_writes(H):
    """A token outside the vocabulary and a context with no room for K+1 new
    positions: accepted/next = -1, ctx unchanged, error bits set, the cache of
    the offending sequence untouched; the other sequences are unaffected."""
    cfg = workloads.scaled(workloads.get_config("tiny_fp32"), batch=3, n_layers=2)
    case = H.Case(cfg)
    run = H.GpuRun(case)
    com = case.committed.clone()
    com[1] = cfg.vocab + 5
    ctx = case.ctx.clone()
    ctx[2] = case.cap - cfg.k_draft          # no room for K+1 positions
    H.say("[errors] bad token in seq 1, capacity overflow in seq 2")
    before = run.kc.clone()
    g = run.step(com, case.rtok[0], ctx)
    assert g["accepted"][1] == -1 and g["next_tok"][1] == -1 and g["ctx_out"][1] == ctx[1]
    assert g["accepted"][2] == -1 and g["ctx_out"][2] == ctx[2]
    assert torch.equal(before[2], run.kc[2])
    word = run.ctx.error_word(clear=True)
    import speculative_decoding_verify_step_amd as sv
    assert word & sv.SV_DEV_BAD_TOKEN and word & sv.SV_DEV_CAPACITY
    assert g["accepted"][0] >= 0 and g["ctx_out"][0] == ctx[0] + g["accepted"][0] + 1
    assert run.ctx.error_word() == 0
    run.close()


def _tiled16_reference(W: torch.Tensor, esize: int) -> torch.Tensor:
    """The documented tiled16 layout built with torch reshapes: rows padded to
    16, block r and step s at KiB (r * steps + s), lane l = (row l%16, slice
    l/16) of the step, KL = 16 / esize elements per slice."""
    rows, cols = W.shape
    KL = 16 // esize
    S = 4 * KL
    pad = (-rows) % 16
    if pad:
        W = torch.cat([W, torch.zeros(pad, cols, dtype=W.dtype, device=W.device)])
    nb = W.shape[0] // 16
    t = W.reshape(nb, 16, cols // S, 4, KL)          # block, row, step, slice, elem
    t = t.permute(0, 2, 3, 1, 4).contiguous()        # block, step, slice, row, elem
    return t.view(torch.uint8).reshape(-1)


@pytest.mark.parametrize("dtype,rows,cols", [("f32", 24, 64), ("bf16", 48, 96), ("fp8", 40, 128),
                                             ("bf16", 1792, 1280)])
def test_pack_tiled16_layout(H, dtype, rows, cols):
    import speculative_decoding_verify_step_amd as sv
    g = torch.Generator(device="cuda").manual_seed(3)
    W = torch.randn(rows, cols, generator=g, device="cuda")
    if dtype == "bf16":
        W = W.to(torch.bfloat16)
    elif dtype == "fp8":
        W = W.to(torch.float8_e4m3fn).view(torch.uint8)
    esize = W.element_size()
    H.say(f"[pack] {dtype} {rows}x{cols}")
    got = sv.pack_matrix(W)
    torch.cuda.synchronize()
    want = _tiled16_reference(W.view(torch.uint8).view(W.dtype) if dtype != "fp8" else W, esize)
    assert got.numel() == want.numel()
    assert torch.equal(got, want)


@pytest.mark.parametrize("batch", [17, 5, 12, 64])
def test_row_major_and_tiled16_layouts_agree_bitwise(H, batch):
    """The two weight layouts feed the same values in the same order to the
    same arithmetic: every output is bit-identical -- at 68 rows (the
    large-row kernels), 20 and 48 rows (two and four row fragments on the
    few-row kernels) and 256 rows (32-row expert tiles)."""
    cfg = workloads.scaled(workloads.get_config("moe_b32"), n_layers=2, vocab=4096, batch=batch,
                           ctx=("uniform", 40, 300))
    case = H.Case(cfg)
    outs = []
    for layout in ("row_major", "tiled16"):
        H.say(f"[layouts] {layout}")
        run = H.GpuRun(case, layout=layout)
        outs.append(run.step(case.committed, case.rtok[0], case.ctx))
        run.close()
    for k in ("logits", "hidden", "target", "accepted", "next_tok", "ctx_out", "routing"):
        assert np.array_equal(outs[0][k], outs[1][k], equal_nan=True), k


@pytest.mark.parametrize("name,overrides", [
    ("tiny_fp32", dict(batch=1)),
    ("tiny_fp32", dict(batch=17, n_q=4, n_kv=4, head_dim=128, ctx=("uniform", 60, 400))),
    ("dense_fp8_b8", dict(n_layers=1, hidden=512, n_q=8, n_kv=2, dense_inter=1024, vocab=4096, batch=2,
                          k_draft=7, ctx=("uniform", 60, 400))),
    ("moe_b1", dict(n_layers=2, hidden=256, n_q=2, n_kv=2, n_experts=16, expert_inter=128, top_k=4,
                    n_shared=1, vocab=2048, batch=3, ctx=("uniform", 1, 200), wdtype="fp8")),
])
def test_layouts_agree_bitwise_fp32_and_fp8(H, name, overrides):
    """The row-major and tiled16 weight layouts bit for bit with fp32 weights
    (4 rows, and 68 rows at head dimension 128) and e4m3 weights (dense at
    16 rows, MoE at 12 rows): the row-major kernels of these dtypes against
    the tiled ones, which the other tests compare with the oracle.  (Above
    64 rows tiled e4m3 weights run the wide-tile kernels with other K
    splits: see the next test.)"""
    cfg = workloads.scaled(workloads.get_config(name), **overrides)
    case = H.Case(cfg)
    outs = []
    for layout in ("row_major", "tiled16"):
        H.say(f"[layouts {cfg.wdtype} T={cfg.batch * (cfg.k_draft + 1)}] {layout}")
        run = H.GpuRun(case, layout=layout)
        outs.append(run.step(case.committed, case.rtok[0], case.ctx))
        run.close()
    for k in ("logits", "hidden", "target", "accepted", "next_tok", "ctx_out", "routing"):
        if outs[1][k] is None:   # routing of a dense model
            assert outs[0][k] is None, k
            continue
        assert np.array_equal(outs[0][k], outs[1][k], equal_nan=True), k


@pytest.mark.parametrize("name,overrides", [
    ("dense_fp8_b8", dict(n_layers=1, hidden=512, n_q=8, n_kv=2, dense_inter=1024, vocab=4096, batch=3,
                          k_draft=31, ctx=("uniform", 60, 400))),
    ("moe_b1", dict(n_layers=2, hidden=256, n_q=2, n_kv=2, n_experts=16, expert_inter=128, top_k=4,
                    n_shared=1, vocab=2048, batch=20, ctx=("uniform", 1, 200), wdtype="fp8")),
])
def test_row_major_fp8_many_rows(H, name, overrides):
    """Row-major e4m3 weights above 64 rows (dense at 96, MoE at 80) run the
    16x16 large-row kernels where the tiled layout runs the wide-tile and
    LDS-staged ones with other K splits (another summation order, so not
    bit-identical): compared with the oracle."""
    cfg = workloads.scaled(workloads.get_config(name), **overrides)
    stats, _ = _verify_case(H, cfg, label=f"fp8_row_major_{cfg.ffn}", layout="row_major")
    assert stats["argmax_agree"] >= 0.8 * stats["positions"]

