"""Benchmark of the greedy speculative-decoding verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--sampled | --draft-loop]

A step is one spec_verify_step over a whole batch (every row of the hot
path: embedding, all decoder layers, LM head + argmax, acceptance + commit).
Inputs are seeded synthetic tensors resident in HBM before timing starts.
Drafts follow the workload's rule (copy the target's greedy token with the
match probability, else a uniform token) and are recorded in untimed passes,
then replayed, so the timed steps accept exactly what was recorded.

Without --config the run covers the metric's three batch points in one
invocation: batch 1 (moe_b1, the line's headline value), batch 32 (moe_b32,
12 layers) and batch 64 (moe_b64_long, 12 layers, its chain of 100 steps).
Single-step workloads cycle through 16 recorded draft sets over K timed
steps (same contexts); the chained workload runs its steps in order, contexts
growing by accepted + 1 and the bonus token becoming the next committed
token, all on the device.

--sampled times the sampled (rejection-sampling) step instead, at temperature
1 with drafts drawn from seeded draft distributions; its line adds the time
of the sampling kernels.  --draft-loop times the device-resident FastMTP
draft -> verify loop (spec_draft_step after every spec_verify_step) and
reports the draft step's share.

One JSON line is printed: accepted tokens/s (sum over sequences of
accepted + 1 per step, over the timed wall clock), microseconds per step
(mean over the timed region; p50 / p90 from an eager re-run with events
between steps), the roofline of the dominant kernel (algorithmic bytes / its
mean duration from HIP events recorded around its launches on the launch
stream), every kernel class's time per step, the whole step against the HBM
roofline, and the CPU oracle's throughput on the host as a reported
baseline; the default run adds a block per batch point under "batches".
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# HBM traffic of each workload's dominant kernel, measured with rocprofv3
# (profiles/hbm_traffic_dominant_kernels.md): bytes read per dispatch =
# 128 TCC_EA0_RDREQ_128B + 64 TCC_EA0_RDREQ_64B + 32 TCC_EA0_RDREQ_32B, bytes
# written = 64 TCC_EA0_WRREQ_64B + 32 (TCC_EA0_WRREQ - TCC_EA0_WRREQ_64B); a
# plain 1 GiB device copy reads and writes exactly 1 GiB by these formulas.
# Median over the dispatches of the same command.  Valid only for the kernel
# sources it was measured on (SHA-256 prefix of every .h / .hip file of the
# library's csrc/, in name order).
MEASURED_TRAFFIC = {   # the dominant kernel of each workload (see DOMINANT)
    "moe_b1": {"source_sha": "5718c341cd100a7d", "read_bytes": 331_100_000, "write_bytes": 65_000},
    "moe_b32": {"source_sha": "5718c341cd100a7d", "read_bytes": 305_513_000, "write_bytes": 1_835_000},
    # the whole 100-step chain (contexts growing as in the benchmark)
    "moe_b64_long": {"source_sha": "5718c341cd100a7d", "read_bytes": 1_604_064_000,
                     "write_bytes": 13_945_000},
    "dense_fp8_b8": {"source_sha": "5718c341cd100a7d", "read_bytes": 124_073_000, "write_bytes": 31_229_000},
}


def kernel_source_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "speculative_decoding_verify_step_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if not f.endswith((".h", ".hip")):
            continue
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    m = MEASURED_TRAFFIC.get(workload)
    if m is None or m["source_sha"] != kernel_source_sha():
        return None
    return m["read_bytes"] + m["write_bytes"]
METRIC = "accepted tokens/s + verify-step µs at batch 1/32/64, K=3, MoE decoder"
WBYTES = {"f32": 4, "bf16": 2, "fp8": 1}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------ byte model
def lm_head_bytes(cfg, T, logits=False):
    """Algorithmic HBM bytes of one LM-head launch: the weight matrix (and
    fp8 row scales) once, the normalised activations once, the argmax
    partial keys written (one 8-byte key per 64-column tile and row), and
    for sampled verification the fp32 logits written."""
    V, H = cfg.vocab, cfg.hidden
    w = V * H * WBYTES[cfg.wdtype] + (V * 4 if cfg.wdtype == "fp8" else 0)
    if cfg.mx == "mxfp4":            # half-byte codes + one scale byte per 32
        w = V * H // 2 + V * H // 32
    act = T * H * (4 if cfg.wdtype == "f32" else 2)
    keys = ((V + 63) // 64) * T * 8
    return w + act + keys + (T * V * 4 if logits else 0)


def step_bytes(cfg, ctx, distinct_experts):
    """Algorithmic bytes of one step: every weight the step needs, once
    (routed experts counted from the actual routing), the cached context read
    once per (sequence, layer, KV head) and the new K/V written."""
    H, D, L = cfg.hidden, cfg.head_dim, cfg.n_layers
    wb = WBYTES[cfg.wdtype]
    sc = 4 if cfg.wdtype == "fp8" else 0
    T = cfg.batch * (cfg.k_draft + 1)
    kvb = 4 if cfg.kvdtype == "f32" else 2
    per_layer = (cfg.qkv_dim * H + H * cfg.n_q * D) * wb + (cfg.qkv_dim + H) * sc
    total = 0
    for l in range(L):
        total += per_layer
        if cfg.ffn == "moe":
            ex = 3 * H * cfg.expert_inter * wb
            if cfg.mx == "mxfp4":
                ex = 3 * H * cfg.expert_inter * 17 // 32     # codes + block scales
            total += cfg.n_experts * H * wb + (distinct_experts[l] + cfg.n_shared) * ex
        else:
            total += 3 * H * cfg.dense_inter * wb + (3 * cfg.dense_inter) * sc
    if cfg.mx == "mxfp4":
        total += cfg.vocab * H * 17 // 32                        # LM head codes + scales
    else:
        total += cfg.vocab * H * wb + cfg.vocab * sc             # LM head
    total += T * H * (4 if cfg.embdtype == "f32" else 2)        # embedding rows
    kv_read = sum(int(c) + cfg.k_draft + 1 for c in ctx) * 2 * cfg.n_kv * D * L * kvb
    kv_write = T * 2 * cfg.n_kv * D * L * kvb
    return total + kv_read + kv_write


def attention_bytes(cfg, ctx_sum_mean):
    """Algorithmic bytes of one split-KV attention launch (one layer): every
    cached and new K/V row of every sequence read once, the queries read once.
    ctx_sum_mean: the sum over sequences of (context + K + 1), averaged over
    the timed steps."""
    kvb = 4 if cfg.kvdtype == "f32" else 2
    T = cfg.batch * (cfg.k_draft + 1)
    return int(ctx_sum_mean * 2 * cfg.n_kv * cfg.head_dim * kvb + T * cfg.n_q * cfg.head_dim * 2)


def gate_up_bytes(cfg, distinct_mean):
    """Algorithmic bytes of one grouped expert gate/up launch (one layer): the
    gate and up rows of every routed expert used and of the shared experts
    once, the normalised rows once, the SwiGLU outputs written once."""
    H, I = cfg.hidden, cfg.expert_inter
    T = cfg.batch * (cfg.k_draft + 1)
    w = (distinct_mean + cfg.n_shared) * 2 * I * H * WBYTES[cfg.wdtype]
    return int(w + T * H * 2 + (T * cfg.top_k + cfg.n_shared * T) * I * 2)


# The kernel class with the largest share of a step (kernel traces): the LM
# head at batch 1; at batch 32 the grouped expert gate/up (742 us of 2,450);
# at batch 64 with long contexts the attention (3,050 of 5,331); dense fp8
# with K = 31 the attention (401 of 2,014).
DOMINANT = {"moe_b32": "expert_gate_up", "moe_b64_long": "attention", "dense_fp8_b8": "attention"}
# kernel classes timed per step in every workload block
CLASSES = ("lm_head", "attention", "expert_gate_up", "expert_down", "qkv")
MFMA_PEAK_TFLOPS = 2500.0     # dense bf16 (fp8 weights are widened to bf16 before the product)
HEADLINE = "moe_b1"           # the batch-1 workload the headline value is quoted on
MULTI = ("moe_b1", "moe_b32", "moe_b64_long")   # the metric's batch 1 / 32 / 64 points
STEP_TARGET_FRAC = 0.60       # the batch-1 step's target fraction of the HBM roofline
N_DRAFT_SETS = 16             # recorded draft sets cycled by single-step workloads


def class_flops(cfg, kclass):
    """Algorithmic flops of one launch of a matrix-product kernel class (2
    per multiply-add; routed experts counted per routed row), or None."""
    T = cfg.batch * (cfg.k_draft + 1)
    H = cfg.hidden
    if kclass == "lm_head":
        return 2 * T * cfg.vocab * H
    if kclass == "qkv":
        return 2 * T * cfg.qkv_dim * H
    if kclass in ("expert_gate_up", "expert_down"):
        if cfg.ffn == "moe":
            rows, inter = T * cfg.top_k + cfg.n_shared * T, cfg.expert_inter
        else:
            rows, inter = T, cfg.dense_inter
        return 2 * rows * inter * H * (2 if kclass == "expert_gate_up" else 1)
    return None


# ------------------------------------------------------------- workload
def setup(cfg, steps, kv_page=0):
    """Weights, caches and a context.  kv_page > 0: the caches live in page
    pools of that many positions, in a seeded random physical order (every
    sequence's pages scattered over the pool)."""
    import numpy as np
    import torch

    import speculative_decoding_verify_step_amd as sv
    import workloads

    cap = workloads.capacity_for(workloads.scaled(cfg, steps=max(cfg.steps, steps)))
    if kv_page:
        cap = (cap + kv_page - 1) // kv_page * kv_page
    w = workloads.make_weights(cfg, "cuda")
    k, v = workloads.kv_cache(cfg, "cuda", capacity=cap)
    k, v = sv.kv_to_library(k, v)
    table = None
    if kv_page:
        n_pages = cfg.batch * cap // kv_page
        order = np.random.default_rng(cfg.seed).permutation(n_pages)
        k, v, table = sv.kv_paged_from_library(k, v, kv_page, order)
    torch.cuda.synchronize()
    ctx = workloads.context_lengths(cfg)
    com = workloads.committed_tokens(cfg)
    n_rec = steps if cfg.steps > 1 else N_DRAFT_SETS
    coins, rtok = workloads.draft_randomness(cfg, steps=n_rec)
    vc = sv.VerifyContext(cfg, cfg.batch, cap, w, kv_page_size=kv_page,
                          kv_pool_pages=k.shape[0] if kv_page else 0)
    if kv_page:
        vc.set_kv_pages(table)
    return dict(sv=sv, w=w, k=k, v=v, cap=cap, ctx=ctx, com=com, coins=coins, rtok=rtok, vc=vc,
                n_rec=n_rec, chained=cfg.steps > 1)


def record_drafts(cfg, S):
    """Drafts of every recorded set (single-step workloads: N_DRAFT_SETS
    independent draw sets on the same start state; chained: one per step of
    the chain) by the workload's rule, the target's tokens taken from untimed
    passes of the library itself; returns per-set device tensors and the
    number of distinct routed experts per layer under each set's routing."""
    import torch
    vc = S["vc"]
    B, K = cfg.batch, cfg.k_draft
    K1 = K + 1
    dev = "cuda"
    i32 = dict(dtype=torch.int32, device=dev)
    target = torch.empty(B, K1, **i32)
    routing = (torch.empty(cfg.n_layers, B * K1, cfg.top_k, **i32) if cfg.ffn == "moe" else None)
    vc.set_debug(None, None, target, routing)
    ctx = S["ctx"].to(**i32)
    com = S["com"].to(**i32)
    tmp_ctx, acc, nxt = (torch.empty(B, **i32) for _ in range(3))
    drafts, distinct = [], []
    for s in range(S["n_rec"]):
        d = S["rtok"][s].to(**i32).clone()
        coin = S["coins"][s].to(dev).bool()
        for i in range(K):
            vc.step(S["k"], S["v"], com, d, ctx, tmp_ctx, acc, nxt)
            d[:, i] = torch.where(coin[:, i], target[:, i], d[:, i])
        drafts.append(d)
        # the set's own pass (routing for the byte model); a chain advances
        vc.step(S["k"], S["v"], com, d, ctx, ctx if S["chained"] else tmp_ctx, acc, nxt)
        if routing is not None:
            distinct.append([int(torch.unique(routing[l]).numel()) for l in range(cfg.n_layers)])
        if S["chained"]:
            com = nxt.clone()
    vc.set_debug(None, None, None, None)
    torch.cuda.synchronize()
    return drafts, distinct


def _pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs), q))


def run_bench(cfg, steps, warmup, sampled=False, kv_page=0, graph=False, classes=True):
    """Times `steps` verify steps of `cfg` (one pass of the whole hot path over
    the batch each) and returns the workload's measurements.  graph: the
    timed steps are captured once into one HIP graph and the timed region is a
    single replay of it (no host work between steps); otherwise eager
    launches.  Single-step workloads cycle through the recorded draft sets;
    a chained workload runs its steps in order, contexts growing by accepted +
    1 on the device.  After the timed region, eager passes of the same steps
    from the same start state give the per-step distribution (HIP events
    between steps) and the time of each kernel class (HIP events riding on
    the class's launches)."""
    import torch

    import workloads

    S = setup(cfg, steps, kv_page)
    sv, vc = S["sv"], S["vc"]
    B, K1 = cfg.batch, cfg.k_draft + 1
    log(f"[bench] {cfg.name}: B={B} L={cfg.n_layers} cap={S['cap']} recording "
        f"{S['n_rec']} draft set(s)")
    drafts, distinct_sets = record_drafts(cfg, S)
    i32 = dict(dtype=torch.int32, device="cuda")
    if sampled:
        # drafts drawn from seeded draft distributions (rejection sampling at
        # temperature 1); a fresh noise offset every step
        sd = workloads.sampled_drafts(cfg)
        sq, su = sd["q"].to("cuda").contiguous(), sd["u"].to("cuda").contiguous()
        drafts = [sd["drafts"].to(**i32).contiguous()]
    ctx0 = S["ctx"].to(**i32)
    com0 = S["com"].to(**i32)
    nxt, cout = (torch.empty(B, **i32) for _ in range(2))
    chained = S["chained"]
    acc_all = torch.empty(max(steps, warmup, 1), B, **i32)
    com_bufs = [com0.clone(), com0.clone()]

    def one(i, ctx):
        # chained: the bonus token of step i is the committed token of step i+1
        # (two alternating buffers, no copy); contexts grow in place
        d = drafts[i % len(drafts)]
        com_in, ctx_out, nxt_out = ((com_bufs[i % 2], ctx, com_bufs[(i + 1) % 2]) if chained
                                    else (com0, cout, nxt))
        if sampled:
            vc.step_sampled(S["k"], S["v"], com_in, d, sq, su, 1.0, sd["seed"], i, ctx, ctx_out,
                            acc_all[i], nxt_out)
        else:
            vc.step(S["k"], S["v"], com_in, d, ctx, ctx_out, acc_all[i], nxt_out)

    ctx = ctx0.clone()

    def restore():
        ctx.copy_(ctx0)
        com_bufs[0].copy_(com0)

    # warmup (untimed); a chained run restarts from the recorded start state
    for i in range(warmup):
        one(i, ctx)
    torch.cuda.synchronize()
    restore()
    dom = "lm_head" if sampled else DOMINANT.get(cfg.name, "lm_head")
    kc_of = {"lm_head": sv.SV_KC_LM_HEAD, "attention": sv.SV_KC_ATTENTION,
             "expert_gate_up": sv.SV_KC_EXPERT_GATE_UP, "expert_down": sv.SV_KC_EXPERT_DOWN,
             "qkv": sv.SV_KC_QKV}
    ktime = {}
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                one(i, ctx)
        restore()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ref = (ctx.clone(), acc_all[:steps].clone())
        del g
    else:
        vc.kernel_time(kc_of[dom], enable=1, query=False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            one(i, ctx)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ktime[dom] = vc.kernel_time(kc_of[dom], enable=0)
        ref = (ctx.clone(), acc_all[:steps].clone())
    acc_t = acc_all[:steps].to(torch.int64).cpu()
    assert vc.error_word() == 0, "device error during the benchmark"
    # per-step times: an eager pass with events between steps; it must
    # reproduce the timed steps' outcome
    per_step_us = [1e6 * (t1 - t0) / steps] * steps     # without the re-run: the mean
    if classes:
        restore()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(steps):
            one(i, ctx)
            ev[i + 1].record()
        torch.cuda.synchronize()
        per_step_us = [1e3 * ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        assert torch.equal(ctx, ref[0]) and torch.equal(acc_all[:steps], ref[1]), \
            "timed and re-run steps disagree"
    # each kernel class in its own eager pass of the same steps
    for name in (CLASSES if classes else (dom,)):
        if name in ktime:
            continue
        restore()
        vc.kernel_time(kc_of[name], enable=1, query=False)
        for i in range(steps):
            one(i, ctx)
        torch.cuda.synchronize()
        ktime[name] = vc.kernel_time(kc_of[name], enable=0)
    assert vc.error_word() == 0, "device error during the benchmark"
    samp_us = None
    if sampled:   # the sampling kernels, timed in a further pass of the same steps
        restore()
        vc.kernel_time(sv.SV_KC_SAMPLING, enable=1, query=False)
        for i in range(steps):
            one(i, ctx)
        torch.cuda.synchronize()
        s_ms, s_n = vc.kernel_time(sv.SV_KC_SAMPLING, enable=0)
        samp_us = 1e3 * s_ms / max(steps, 1)
    wall = t1 - t0
    committed_tokens = int(acc_t.sum().item()) + steps * B
    ms_step = wall * 1e3 / steps
    # contexts of every timed step: the start plus the commits before it
    c0 = ctx0.to(torch.int64).cpu()
    if chained:
        grown = torch.cumsum(acc_t + 1, 0) - (acc_t + 1)
        ctx_steps = c0.unsqueeze(0) + grown               # [steps][B]
    else:
        ctx_steps = c0.unsqueeze(0).expand(steps, B)
    ctx_sum_mean = float((ctx_steps + K1).sum(1).double().mean())
    nsets = len(drafts)
    sb = []
    for i in range(steps):
        dist = distinct_sets[i % nsets] if distinct_sets else [0] * cfg.n_layers
        sb.append(step_bytes(cfg, ctx_steps[i].tolist(), dist))
    step_b = sum(sb) / len(sb)
    if distinct_sets:
        dmean = [sum(distinct_sets[i % nsets][l] for i in range(steps)) / steps
                 for l in range(cfg.n_layers)]
    else:
        dmean = []
    if dom == "lm_head":
        kbytes = lm_head_bytes(cfg, B * K1, logits=sampled)
    elif dom == "attention":
        kbytes = attention_bytes(cfg, ctx_sum_mean)
    else:
        kbytes = gate_up_bytes(cfg, sum(dmean) / len(dmean))
    kernels = {}
    for name, (ms, n) in ktime.items():
        if n == 0:
            continue
        ent = {"mean_us": 1e3 * ms / n, "launches_per_step": n / steps,
               "us_per_step": 1e3 * ms / steps}
        fl = class_flops(cfg, name)
        if fl is not None:
            tf = fl / (ms / n * 1e-3) / 1e12
            ent["tflops"] = tf
            ent["mfma_frac"] = tf / MFMA_PEAK_TFLOPS
        if name == "attention":
            ent["GBs"] = attention_bytes(cfg, ctx_sum_mean) / (ms / n * 1e-3) / 1e9
        if name == "lm_head":
            ent["GBs"] = lm_head_bytes(cfg, B * K1, logits=sampled) / (ms / n * 1e-3) / 1e9
        kernels[name] = ent
    dom_ms, dom_n = ktime[dom]
    res = {
        "ms_per_step": ms_step,
        "p50_us": _pct(per_step_us, 50),
        "p90_us": _pct(per_step_us, 90),
        "tok_s": committed_tokens / wall,
        "tau": committed_tokens / (steps * B),
        "draft_sets": nsets,
        "kernel": dom,
        "lm_ms": dom_ms / max(dom_n, 1),
        "lm_launches": dom_n,
        "lm_bytes": kbytes,
        "sampling_us_per_step": samp_us,
        "step_bytes": step_b,
        "distinct_experts": [round(x, 2) for x in dmean],
        "kernels": kernels,
        "ctx_end": ctx.tolist() if chained else None,
        "weights": S["w"],
        "cap": S["cap"],
    }
    vc.close()
    return res


def attention_kernel(cfg):
    """The library's attention kernel for cfg: the LDS-ring kernel when a KV
    head has 17 .. 256 query rows (block positions x grouped query heads) and
    the cache is bf16, else the split-KV kernel."""
    rows = (cfg.k_draft + 1) * (cfg.n_q // cfg.n_kv)
    return "attn_lds" if cfg.kvdtype == "bf16" and 17 <= rows <= 256 else "attn_split"


def block(cfg, r, steps, graph, sampled=False, kv_page=0):
    """The JSON object of one workload's measurements."""
    lm_gbs = r["lm_bytes"] / (r["lm_ms"] * 1e-3) / 1e9 if r["lm_ms"] > 0 else None
    step_gbs = r["step_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9
    return {
        "workload": cfg.name, "batch": cfg.batch, "k_draft": cfg.k_draft, "layers": cfg.n_layers,
        "steps": steps, "chained_steps": cfg.steps > 1,
        "launch": "one HIP graph of all timed steps" if graph else "eager",
        "us_per_step": r["ms_per_step"] * 1e3, "p50_us": r["p50_us"], "p90_us": r["p90_us"],
        "accepted_tok_s": r["tok_s"], "tokens_per_verify": r["tau"],
        "draft_sets": r["draft_sets"],
        "roofline": {"bound": "hbm",
                     "kernel": {"lm_head": "lm_head_argmax", "attention": attention_kernel(cfg),
                                "expert_gate_up": "expert_gate_up_swiglu"}[r["kernel"]],
                     "achieved": lm_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": (lm_gbs / HBM_PEAK_GBS) if lm_gbs else None,
                     "traffic": (None if sampled or kv_page else measured_traffic(cfg.name)),
                     "mean_us": r["lm_ms"] * 1e3, "bytes_per_launch": r["lm_bytes"],
                     "launches_timed": r["lm_launches"]},
        "step_roofline": {"bytes_per_step": r["step_bytes"], "achieved_GBs": step_gbs,
                          "frac": step_gbs / HBM_PEAK_GBS,
                          "distinct_experts_per_layer": r["distinct_experts"]},
        "kernels": r["kernels"],
        **({"sampling_us_per_step": r["sampling_us_per_step"]} if sampled else {}),
    }


def run_draft_loop(cfg, steps, warmup, graph=False):
    """The device-resident draft -> verify loop: every iteration verifies the
    current drafts (spec_verify_step) and lets the FastMTP draft head propose
    the next ones (spec_draft_step) from the verify step's outcome; contexts
    grow by accepted + 1 and the bonus token becomes the next committed token,
    all on the device.  Seeded random weights for the target and the draft
    head, so drafts are rarely accepted: the line measures cost, not the
    pages' acceptance.  graph: the timed iterations are captured once into
    one HIP graph and replayed; an eager re-run of the same iterations from
    the same state (events around the drafting) must give the same accepted
    lengths and contexts."""
    import torch

    import speculative_decoding_verify_step_amd as sv
    import workloads

    K1 = cfg.k_draft + 1
    n_it = warmup + 2 * steps
    c_loop = workloads.scaled(cfg, steps=n_it)
    cap = workloads.capacity_for(c_loop) + 64
    w = workloads.make_weights(cfg, "cuda")
    k, v = workloads.kv_cache(cfg, "cuda", capacity=cap)
    k, v = sv.kv_to_library(k, v)
    vc = sv.VerifyContext(cfg, cfg.batch, cap, w)
    mc = workloads.mtp_config(cfg)
    mw = workloads.mtp_weights(cfg, "cuda")
    mk, mv = workloads.kv_cache(mc, "cuda", capacity=cap)
    mk, mv = sv.kv_to_library(mk, mv)
    dc = sv.DraftContext(mc, cfg.batch, cap, vc.weights, mw)
    B = cfg.batch
    i32 = dict(dtype=torch.int32, device="cuda")
    ctx0 = workloads.context_lengths(cfg).to(**i32)
    com0 = workloads.committed_tokens(cfg).to(**i32)
    _, rtok = workloads.draft_randomness(cfg, steps=1)
    d0 = rtok[0].to(**i32).contiguous()
    ctxs = [ctx0.clone(), ctx0.clone()]
    coms = [com0.clone(), com0.clone()]
    drs = [d0.clone(), d0.clone()]
    acc_all = torch.empty(n_it, B, **i32)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_it)]

    def one(i, timed):
        a, b_ = i % 2, (i + 1) % 2
        vc.step(k, v, coms[a], drs[a], ctxs[a], ctxs[b_], acc_all[i], coms[b_])
        if timed:
            ev[i][0].record()
        dc.draft(mk, mv, vc, ctxs[a], acc_all[i], coms[b_], drs[a], drs[b_])
        if timed:
            ev[i][1].record()

    for i in range(warmup):
        one(i, False)
    torch.cuda.synchronize()
    timed_its = range(warmup, warmup + steps)
    if graph:
        state = [t.clone() for t in ctxs + coms + drs + [k, v, mk, mv]]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in timed_its:
                one(i, False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        acc_graph = acc_all[warmup:warmup + steps].clone()
        end_graph = [t.clone() for t in ctxs + coms + drs]
        for t, s0 in zip(ctxs + coms + drs + [k, v, mk, mv], state):
            t.copy_(s0)
        del state, g
        for i in timed_its:   # the same iterations, eager, with events around the drafts
            one(i, True)
        torch.cuda.synchronize()
        assert torch.equal(acc_all[warmup:warmup + steps], acc_graph), "graph replay differs"
        assert all(torch.equal(a_, b2) for a_, b2 in zip(ctxs + coms + drs, end_graph)), \
            "graph replay differs"
        draft_ms = sum(ev[i][0].elapsed_time(ev[i][1]) for i in timed_its) / steps
    else:
        t0 = time.perf_counter()
        for i in timed_its:
            one(i, False)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        for i in range(warmup + steps, n_it):   # a second pass with events around the drafts
            one(i, True)
        torch.cuda.synchronize()
        draft_ms = sum(ev[i][0].elapsed_time(ev[i][1]) for i in range(warmup + steps, n_it)) / steps
    assert vc.error_word() == 0 and dc.error_word() == 0, "device error during the loop"
    acc = acc_all[warmup:warmup + steps].to(torch.int64)
    tok = int(acc.sum().item()) + steps * B
    res = {"ms_per_step": wall * 1e3 / steps, "tok_s": tok / wall, "tau": tok / (steps * B),
           "draft_ms": draft_ms}
    dc.close()
    vc.close()
    return res


# ----------------------------------------------------------- CPU baseline
def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _host_tree(w):
    import torch
    if isinstance(w, dict):
        return {k: _host_tree(v) for k, v in w.items()}
    if isinstance(w, list):
        return [_host_tree(v) for v in w]
    return w.cpu() if isinstance(w, torch.Tensor) else w


def cpu_baseline(cfg, budget_s=15.0, weights=None, min_steps=3):
    """The oracle, as it is, on this host: whole verify steps of sequence 0
    of the workload (the same shapes and seeds; drafts by the workload's rule
    through the oracle), repeated until about `budget_s` seconds of work (at
    least `min_steps`).  `weights`: the workload's weight dict (any device;
    copied to the host), else generated on the host."""
    import oracle
    import workloads

    c1 = workloads.scaled(cfg, batch=1)
    cap = workloads.capacity_for(cfg)
    w = _host_tree(weights) if weights is not None else workloads.make_weights(c1, "cpu")
    k, v = workloads.kv_cache(c1, "cpu", capacity=cap)
    orc = oracle.Oracle(c1, w, cap)
    kc, vc = orc.kv_np(k, v)
    del k, v
    ctx = int(workloads.context_lengths(cfg)[0])
    com = int(workloads.committed_tokens(cfg)[0])
    coins, rtok = workloads.draft_randomness(cfg, steps=1)
    d = orc.make_drafts(kc, vc, 0, ctx, com, coins[0, 0], rtok[0, 0])
    n, tok, t0 = 0, 0, time.perf_counter()
    while True:
        out = orc.verify_step(kc, vc, [com], d[None], [ctx])
        tok += int(out["accepted"][0]) + 1
        n += 1
        el = time.perf_counter() - t0
        if (el >= budget_s and n >= min_steps) or n >= 200:
            break
    return {"value": tok / el, "unit": "tokens/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{n} whole verify steps of one sequence of {cfg.name} "
                      f"(ctx {ctx}, K={cfg.k_draft}, {cfg.n_layers} layer(s)), "
                      f"{el:.1f} s; per-step {1e3 * el / n:.1f} ms"}


def copy_calibration(nbytes: int, reps: int):
    """A plain device-to-device copy of `nbytes`, `reps` times: the reference
    against which HBM byte counters (FETCH_SIZE, WRITE_SIZE) are scaled --
    each copy must read and write exactly nbytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def _line(cfg, r, steps, warmup, graph, args, blk):
    """The top-level JSON object for one workload."""
    out = {
        "metric": METRIC,
        "value": r["tok_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": r["ms_per_step"],
        "us_per_step": r["ms_per_step"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16+mxfp4" if cfg.mx == "mxfp4" else
                  ("bf16" if cfg.wdtype == "bf16" else cfg.wdtype)),
        "data": "synthetic (seeded N(0,0.02) weights, seeded KV cache and drafts)",
        "config": {"workload": cfg.name, "batch": cfg.batch, "k_draft": cfg.k_draft,
                   "layers": cfg.n_layers, "hidden": cfg.hidden, "vocab": cfg.vocab,
                   "ctx": list(cfg.ctx), "chained_steps": cfg.steps > 1,
                   "weight_layout": "tiled16",
                   "kv": (f"paged ({args.kv_page} positions per page)" if args.kv_page
                          else "contiguous"),
                   "launch": blk["launch"],
                   "verification": "sampled (temperature 1)" if args.sampled else "greedy",
                   "tokens_per_verify": r["tau"], "draft_sets": r["draft_sets"]},
        "roofline": blk["roofline"],
        "step_roofline": dict(blk["step_roofline"]),
        "p50_us": blk["p50_us"],
        "p90_us": blk["p90_us"],
        "kernels": blk["kernels"],
        **({"sampling_us_per_step": blk["sampling_us_per_step"]} if "sampling_us_per_step" in blk else {}),
    }
    if cfg.name == HEADLINE and not args.sampled and not args.kv_page:
        # the batch-1 target applies to the whole step, not to one kernel
        out["step_roofline"]["target_frac"] = STEP_TARGET_FRAC
        out["step_roofline"]["meets_target"] = out["step_roofline"]["frac"] >= STEP_TARGET_FRAC
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps of single-step workloads (a chained workload runs its "
                         "own number of steps)")
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", default=None,
                    help="one workload; default: batch 1, 32 and 64 (moe_b1, moe_b32, "
                         "moe_b64_long) in one line, quoted on batch 1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sampled", action="store_true",
                    help="time the sampled (rejection-sampling) verify step instead of the greedy one")
    ap.add_argument("--draft-loop", action="store_true",
                    help="time the device-resident FastMTP draft -> verify loop")
    ap.add_argument("--kv-page", type=int, default=0, metavar="P",
                    help="paged KV caches: pages of P positions in a shuffled pool")
    ap.add_argument("--graph", action="store_true",
                    help="capture the timed steps into one HIP graph and time its replay "
                         "(the default for single-step workloads)")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from the host (the default for chained workloads)")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="skip the untimed re-runs that give p50/p90 and the per-class kernel "
                         "times (profiler runs)")
    ap.add_argument("--chain-steps", type=int, default=None, metavar="N",
                    help="steps of a chained workload (default: the workload's own, 100)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps or 5)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "libspecverify runs the verify step on one GPU; "
                                   "--gpus must be 1", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import workloads
    warmup = args.warmup if args.warmup is not None else 10

    def steps_of(cfg):
        if cfg.steps > 1:
            return args.chain_steps or cfg.steps
        return args.steps if args.steps is not None else 200

    def graph_of(cfg):
        # short independent steps measured faster replayed from one graph
        # (batch 1, same box, alternating: 118.0 -> 113.4 us; the batch-1
        # draft loop 434.6 -> 434.0 us); long chained steps measured faster
        # with eager launches (graph nodes add about 1 us per kernel there)
        return args.graph or (cfg.steps == 1 and not args.eager)

    if args.draft_loop:
        cfg = workloads.get_config(args.config or HEADLINE)
        steps = args.steps if args.steps is not None else (cfg.steps if cfg.steps > 1 else 200)
        graph = graph_of(cfg)
        r = run_draft_loop(cfg, steps, warmup, graph=graph)
        print(json.dumps({
            "metric": METRIC, "value": r["tok_s"], "unit": "tokens/s", "n_gpus": 1,
            "steps": steps, "warmup": warmup, "ms_per_step": r["ms_per_step"],
            "us_per_step": r["ms_per_step"] * 1e3, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16" if cfg.wdtype == "bf16" else cfg.wdtype,
            "data": "synthetic (seeded random target and draft-head weights)",
            "config": {"workload": cfg.name, "batch": cfg.batch, "k_draft": cfg.k_draft,
                       "mode": "FastMTP draft -> verify loop", "tokens_per_verify": r["tau"],
                       "launch": "one HIP graph of all timed iterations" if graph else "eager"},
            "draft_us_per_step": r["draft_ms"] * 1e3}), flush=True)
        return

    names = [args.config] if args.config else list(MULTI)
    blocks, head = {}, None
    for name in names:
        cfg = workloads.get_config(name)
        steps, graph = steps_of(cfg), graph_of(cfg)
        r = run_bench(cfg, steps, warmup, sampled=args.sampled, kv_page=args.kv_page, graph=graph,
                      classes=not args.no_breakdown)
        blk = block(cfg, r, steps, graph, args.sampled, args.kv_page)
        log(f"[bench] {name}: {blk['us_per_step']:.1f} us/step, "
            f"{blk['accepted_tok_s']:.0f} tok/s, tau {blk['tokens_per_verify']:.3f}")
        if not args.no_cpu_baseline and not args.sampled:
            log(f"[bench] timing the CPU oracle on {name}")
            blk["cpu_baseline"] = cpu_baseline(cfg, 15.0 if name == names[0] else 8.0,
                                               weights=r["weights"])
        if head is None:
            head = _line(cfg, r, steps, warmup, graph, args, blk)
            if "cpu_baseline" in blk:
                head["cpu_baseline"] = blk["cpu_baseline"]
        blocks[str(cfg.batch) if not args.config else cfg.name] = blk
        del r
        torch.cuda.empty_cache()
    if not args.config:
        head["batches"] = blocks
    print(json.dumps(head), flush=True)


if __name__ == "__main__":
    main()
