"""Shared machinery of the GPU parity tests: one seeded case, run through the
HIP library (via its binding) and through the CPU oracle, and the comparison
rules.

Comparison rules (float tolerance `tol` = 2e-2 for bf16 weights, 5e-2 for fp8
weights, 1e-4 for the fp32 workload):
  * logits of every verified position: max |gpu - oracle| <= tol * (max - min of
    the oracle's logits at that position);
  * residual stream after every layer: the same rule against the oracle
    vector's own range;
  * greedy token: bit-exact at every position whose oracle top-2 margin (in
    fp32) exceeds tol * range (the stated-tolerance rule), and also at every
    position whose margin exceeds twice the largest logit error measured at
    that position (the measured-error rule: with every GPU logit within e of
    the oracle's, a margin above 2e cannot flip the argmax, since the GPU's
    argmax is taken on exactly the logits it reports);
  * accepted length, bonus token, new context length: bit-exact for every
    sequence whose deciding positions 0 .. min(a, K) all qualify, under each
    rule;
  * new cache entries: within tol of the oracle's range at every written slot;
  * expert routing (MoE): the GPU reports its router logits; (1) they must lie
    within ROUTER_TOL * (range of the oracle's router logits) of the oracle's,
    element by element; (2) the GPU's experts must be the top-k of its own
    logits; (3) the oracle is then run with the GPU's routing forced, so both
    sides follow one trajectory, and wherever the GPU's choice differs from
    the oracle's own top-k, the oracle-logit gap between the oracle's k-th
    expert and the GPU's weakest one must be at most twice the router-logit
    error measured on that row -- the only way two experts' order can swap
    when every logit is off by at most that error.  The number of such forced
    decisions is counted and capped per test.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import speculative_decoding_verify_step_amd as sv
import workloads

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 5e-2}
# element-wise bound on the router logits, relative to the row's oracle range
ROUTER_TOL = dict(TOL)
# forced routing decisions allowed per test: a fraction of all decisions + 2
FORCED_CAP = 0.10


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _cpu_tree(w):
    if isinstance(w, dict):
        return {k: _cpu_tree(v) for k, v in w.items()}
    if isinstance(w, list):
        return [_cpu_tree(v) for v in w]
    if isinstance(w, torch.Tensor):
        return w.cpu()
    return w


class Case:
    """Inputs of one workload, generated on the GPU once and copied to the
    host for the oracle."""

    def __init__(self, cfg, capacity: int | None = None):
        self.cfg = cfg
        self.cap = capacity or workloads.capacity_for(cfg)
        self.w_gpu = workloads.make_weights(cfg, "cuda")
        self.k_nat, self.v_nat = workloads.kv_cache(cfg, "cuda", capacity=self.cap)
        self.ctx = workloads.context_lengths(cfg)
        self.committed = workloads.committed_tokens(cfg)
        self.coins, self.rtok = workloads.draft_randomness(cfg)
        self._orc = None

    def oracle(self) -> oracle.Oracle:
        if self._orc is None:
            self._orc = oracle.Oracle(self.cfg, _cpu_tree(self.w_gpu), self.cap)
        return self._orc

    def oracle_kv(self, b: int, k=None, v=None):
        """numpy copies of sequence b's caches (natural layout), from the
        given GPU caches (default: the initial ones)."""
        k = self.k_nat if k is None else k
        v = self.v_nat if v is None else v
        return self.oracle().kv_np(k[b:b + 1], v[b:b + 1])

    def drafts(self, sampled, step=0, committed=None, ctx=None, kv=None):
        """Drafts [B][K]: the workload's rule (through the oracle) for the
        sampled sequences, the fallback tokens for the others."""
        cfg = self.cfg
        committed = self.committed if committed is None else committed
        ctx = self.ctx if ctx is None else ctx
        d = self.rtok[step].clone()
        for b in sampled:
            kc, vc = kv[b] if kv is not None else self.oracle_kv(b)
            d[b] = torch.from_numpy(self.oracle().make_drafts(
                kc, vc, 0, int(ctx[b]), int(committed[b]), self.coins[step, b],
                self.rtok[step, b]))
        return d


class GpuRun:
    """One library context with debug outputs for a case."""

    def __init__(self, case: Case, batch: int | None = None, debug=True, layout="tiled16"):
        cfg = case.cfg
        self.case = case
        self.B = cfg.batch if batch is None else batch
        self.ctx = sv.VerifyContext(cfg, self.B, case.cap, case.w_gpu, layout=layout)
        self.kc, self.vc = sv.kv_to_library(case.k_nat[: self.B], case.v_nat[: self.B])
        K1 = cfg.k_draft + 1
        T = self.B * K1
        dev = "cuda"
        self.logits = torch.full((self.B, K1, cfg.vocab), float("nan"), device=dev) if debug else None
        self.hidden = torch.full((cfg.n_layers, T, cfg.hidden), float("nan"), device=dev) if debug else None
        self.target = torch.full((self.B, K1), -7, dtype=torch.int32, device=dev)
        self.routing = (torch.full((cfg.n_layers, T, cfg.top_k), -1, dtype=torch.int32, device=dev)
                        if cfg.ffn == "moe" else None)
        self.rlogits = (torch.full((cfg.n_layers, T, cfg.n_experts), float("nan"), device=dev)
                        if cfg.ffn == "moe" else None)
        self.ctx.set_debug(self.logits, self.hidden, self.target, self.routing)
        if self.rlogits is not None:
            self.ctx.set_debug_router(self.rlogits)
        self.acc = torch.full((self.B,), -9, dtype=torch.int32, device=dev)
        self.nxt = torch.full((self.B,), -9, dtype=torch.int32, device=dev)
        self.ctx_out = torch.full((self.B,), -9, dtype=torch.int32, device=dev)

    def step(self, committed, drafts, ctx_in, ctx_out=None):
        dev = "cuda"
        com = committed.to(dev, torch.int32).contiguous()
        dr = drafts.to(dev, torch.int32).contiguous()
        ci = ctx_in.to(dev, torch.int32).contiguous() if not ctx_in.is_cuda else ctx_in
        co = self.ctx_out if ctx_out is None else ctx_out
        self.ctx.step(self.kc, self.vc, com, dr, ci, co, self.acc, self.nxt, batch=self.B)
        torch.cuda.synchronize()
        return {"accepted": self.acc.cpu().numpy(), "next_tok": self.nxt.cpu().numpy(),
                "ctx_out": co.cpu().numpy(), "target": self.target.cpu().numpy(),
                "logits": None if self.logits is None else self.logits.cpu().numpy(),
                "hidden": None if self.hidden is None else self.hidden.cpu().numpy(),
                "routing": None if self.routing is None else self.routing.cpu().numpy(),
                "rlogits": None if self.rlogits is None else self.rlogits.cpu().numpy()}

    def routing_of(self, g: dict, b: int):
        """The GPU's expert choice for sequence b as [1][L][K+1][top_k] (MoE)."""
        if g["routing"] is None:
            return None
        K1 = self.case.cfg.k_draft + 1
        return g["routing"][:, b * K1:(b + 1) * K1][None]

    def rlogits_of(self, g: dict, b: int):
        """The GPU's router logits for sequence b as [L][K+1][E] (MoE)."""
        if g.get("rlogits") is None:
            return None
        K1 = self.case.cfg.k_draft + 1
        return g["rlogits"][:, b * K1:(b + 1) * K1]

    def close(self):
        self.ctx.close()


def margin_ok(lo: np.ndarray, tol: float) -> bool:
    lf = lo.astype(np.float32)
    top = np.partition(lf, -2)[-2:]
    rng = float(lo.max() - lo.min())
    return float(top[1] - top[0]) > tol * rng


def margin_measured_ok(lo: np.ndarray, err: float) -> bool:
    """True when the oracle's top-2 gap exceeds twice the measured logit error
    (on fp64 values, and still positive after rounding to fp32, where the
    oracle takes its argmax)."""
    top = np.partition(lo, -2)[-2:]
    lf = lo.astype(np.float32)
    top32 = np.partition(lf, -2)[-2:]
    return float(top[1] - top[0]) > 2.0 * err * (1.0 + 1e-6) and float(top32[1] - top32[0]) > 0.0


def compare_sequence(cfg, g: dict, b: int, o: dict, i: int, stats: dict, check_hidden=True):
    """Compare GPU sequence b with oracle output row i under the rules above."""
    tol = TOL[cfg.wdtype]
    K = cfg.k_draft
    K1 = K + 1
    qual, qual_m = [], []
    for j in range(K1):
        lo = o["logits"][i, j]
        lg = g["logits"][b, j].astype(np.float64)
        rng = float(lo.max() - lo.min())
        err = float(np.abs(lg - lo).max())
        stats["max_rel_logit_err"] = max(stats.get("max_rel_logit_err", 0.0), err / rng)
        assert err <= tol * rng, f"seq {b} pos {j}: logit err {err:.3e} > {tol} * range {rng:.3e}"
        q = margin_ok(lo, tol)
        qm = margin_measured_ok(lo, err)
        qual.append(q)
        qual_m.append(qm)
        stats["positions"] = stats.get("positions", 0) + 1
        stats["qualified"] = stats.get("qualified", 0) + int(q)
        stats["qualified_measured"] = stats.get("qualified_measured", 0) + int(qm)
        same = int(g["target"][b, j]) == int(o["target"][i, j])
        stats["argmax_agree"] = stats.get("argmax_agree", 0) + int(same)
        if q or qm:
            assert same, (f"seq {b} pos {j}: argmax {g['target'][b, j]} vs {o['target'][i, j]} "
                          f"(stated rule {q}, measured rule {qm}, err {err:.3e})")
    if check_hidden and "layer_hidden" in o:
        for l in range(cfg.n_layers):
            for j in range(K1):
                ho = o["layer_hidden"][i, l, j]
                hg = g["hidden"][l, b * K1 + j].astype(np.float64)
                rng = float(ho.max() - ho.min())
                err = float(np.abs(hg - ho).max())
                stats["max_rel_hidden_err"] = max(stats.get("max_rel_hidden_err", 0.0), err / rng)
                assert err <= tol * rng, f"seq {b} layer {l} pos {j}: hidden err {err:.3e}"
    a_or = int(o["accepted"][i])
    deciding = range(0, min(a_or, K) + 1)
    stats["sequences"] = stats.get("sequences", 0) + 1
    same_acc = int(g["accepted"][b]) == a_or and int(g["next_tok"][b]) == int(o["next_tok"][i])
    stats["accept_agree"] = stats.get("accept_agree", 0) + int(same_acc)
    stated = all(qual[j] for j in deciding)
    measured = all(qual_m[j] for j in deciding)
    if stated:
        stats["accept_checked"] = stats.get("accept_checked", 0) + 1
    if measured:
        stats["accept_checked_measured"] = stats.get("accept_checked_measured", 0) + 1
    if stated or measured:
        assert int(g["accepted"][b]) == a_or, f"seq {b}: accepted {g['accepted'][b]} vs {a_or}"
        assert int(g["next_tok"][b]) == int(o["next_tok"][i])
        assert int(g["ctx_out"][b]) == int(o["ctx_out"][i])
    return same_acc


def compare_new_kv(cfg, run: GpuRun, b: int, kc_or, vc_or, ctx_b: int, stats: dict):
    """The K+1 slots the step wrote, every layer, against the oracle's cache."""
    tol = TOL[cfg.wdtype]
    K1 = cfg.k_draft + 1
    kn, vn = sv.kv_from_library(run.kc[b:b + 1], run.vc[b:b + 1])
    kg = kn[0, :, :, ctx_b:ctx_b + K1].float().cpu().numpy()
    vg = vn[0, :, :, ctx_b:ctx_b + K1].float().cpu().numpy()
    conv = (lambda a: a.astype(np.float64)) if cfg.kvdtype == "f32" else (
        lambda a: (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    ko = conv(kc_or[0, :, :, ctx_b:ctx_b + K1])
    vo = conv(vc_or[0, :, :, ctx_b:ctx_b + K1])
    for name, gg, oo in (("k", kg, ko), ("v", vg, vo)):
        rng = float(oo.max() - oo.min())
        err = float(np.abs(gg - oo).max())
        stats[f"max_rel_{name}_err"] = max(stats.get(f"max_rel_{name}_err", 0.0), err / rng)
        assert err <= tol * rng, f"seq {b}: new {name} cache err {err:.3e} > {tol} * {rng:.3e}"


def check_routing(cfg, forced: np.ndarray, o: dict, stats: dict, label="", rl_gpu=None):
    """forced [1][L][K+1][k]: the GPU's routing; rl_gpu [L][K+1][E]: the
    GPU's router logits; o: the oracle run with that routing forced
    (want_routing=True)."""
    if forced is None:
        return
    assert rl_gpu is not None, "MoE parity needs the GPU's router logits"
    rtol = ROUTER_TOL[cfg.wdtype]
    rl = o["router_logits"][0]
    L, K1, k = forced.shape[1:]
    for l in range(L):
        for j in range(K1):
            r = rl[l, j]
            rg = rl_gpu[l, j].astype(np.float64)
            gsel = [int(e) for e in forced[0, l, j]]
            assert len(set(gsel)) == k and min(gsel) >= 0 and max(gsel) < cfg.n_experts, (
                f"{label} layer {l} pos {j}: invalid routing {gsel}")
            # (1) router logits element by element
            rng = float(r.max() - r.min())
            err = float(np.abs(rg - r).max())
            stats["max_rel_router_err"] = max(stats.get("max_rel_router_err", 0.0), err / rng)
            assert err <= rtol * rng, (f"{label} layer {l} pos {j}: router logit err {err:.3e} > "
                                       f"{rtol} * range {rng:.3e}")
            # (2) the GPU's experts are the top-k of its own logits, in rank
            # order (fp32 probabilities may tie logits closer than 1e-5)
            rest = [e for e in range(cfg.n_experts) if e not in gsel]
            assert min(rg[gsel]) >= max(rg[rest]) - 1e-5, (
                f"{label} layer {l} pos {j}: GPU experts {gsel} are not the top-{k} of its logits")
            assert all(rg[gsel[q]] >= rg[gsel[q + 1]] - 1e-5 for q in range(k - 1)), (
                f"{label} layer {l} pos {j}: GPU rank order {gsel}")
            stats["routings"] = stats.get("routings", 0) + 1
            # (3) a choice that differs from the oracle's own is a near-tie
            # within twice the measured error of this row
            own = [int(e) for e in oracle.topk(oracle.softmax(r), k)]
            if set(own) == set(gsel):
                continue
            kth = min(r[e] for e in own)
            worst = min(r[e] for e in gsel)
            band = 2.0 * err * (1.0 + 1e-6) + 1e-12
            stats["routing_forced"] = stats.get("routing_forced", 0) + 1
            assert kth - worst <= band, (
                f"{label} layer {l} pos {j}: GPU experts {sorted(gsel)} vs oracle {sorted(own)}, "
                f"oracle-logit gap {kth - worst:.3e} > twice the measured router error {err:.3e}")


def assert_forced_cap(stats: dict, label=""):
    """Forced routing decisions (near-ties) within the cap; printed."""
    n, f = stats.get("routings", 0), stats.get("routing_forced", 0)
    say(f"[{label}] routing decisions {n}, forced {f}, "
        f"max router err {stats.get('max_rel_router_err', 0.0):.2e} of range")
    assert f <= FORCED_CAP * n + 2, f"{label}: {f} forced routing decisions of {n}"
