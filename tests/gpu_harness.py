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
    fp32) exceeds tol * range;
  * accepted length, bonus token, new context length: bit-exact for every
    sequence whose deciding positions 0 .. min(a, K) all pass the margin test;
  * new cache entries: within tol of the oracle's range at every written slot;
  * expert routing (MoE): the oracle is run with the GPU's routing forced, so
    both sides follow one trajectory; the GPU's choice must equal the oracle's
    own top-k wherever the k-th / (k+1)-th router-logit gap exceeds
    tol * (range of the router logits), and elsewhere every expert it chose
    must lie within that band of the oracle's k-th logit.  A near-tie in the
    router is a decision on which both choices are correct to the precision
    of the arithmetic (bf16 activations), so only the band is checked there.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import speculative_decoding_verify_step_amd as sv
import workloads

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 5e-2}


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
        self.ctx.set_debug(self.logits, self.hidden, self.target, self.routing)
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
                "routing": None if self.routing is None else self.routing.cpu().numpy()}

    def routing_of(self, g: dict, b: int):
        """The GPU's expert choice for sequence b as [1][L][K+1][top_k] (MoE)."""
        if g["routing"] is None:
            return None
        K1 = self.case.cfg.k_draft + 1
        return g["routing"][:, b * K1:(b + 1) * K1][None]

    def close(self):
        self.ctx.close()


def margin_ok(lo: np.ndarray, tol: float) -> bool:
    lf = lo.astype(np.float32)
    top = np.partition(lf, -2)[-2:]
    rng = float(lo.max() - lo.min())
    return float(top[1] - top[0]) > tol * rng


def compare_sequence(cfg, g: dict, b: int, o: dict, i: int, stats: dict, check_hidden=True):
    """Compare GPU sequence b with oracle output row i under the rules above."""
    tol = TOL[cfg.wdtype]
    K = cfg.k_draft
    K1 = K + 1
    qual = []
    for j in range(K1):
        lo = o["logits"][i, j]
        lg = g["logits"][b, j].astype(np.float64)
        rng = float(lo.max() - lo.min())
        err = float(np.abs(lg - lo).max())
        stats["max_rel_logit_err"] = max(stats.get("max_rel_logit_err", 0.0), err / rng)
        assert err <= tol * rng, f"seq {b} pos {j}: logit err {err:.3e} > {tol} * range {rng:.3e}"
        q = margin_ok(lo, tol)
        qual.append(q)
        stats["positions"] = stats.get("positions", 0) + 1
        stats["qualified"] = stats.get("qualified", 0) + int(q)
        same = int(g["target"][b, j]) == int(o["target"][i, j])
        stats["argmax_agree"] = stats.get("argmax_agree", 0) + int(same)
        if q:
            assert same, f"seq {b} pos {j}: argmax {g['target'][b, j]} vs {o['target'][i, j]}"
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
    if all(qual[j] for j in deciding):
        stats["accept_checked"] = stats.get("accept_checked", 0) + 1
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


def check_routing(cfg, forced: np.ndarray, o: dict, stats: dict, label=""):
    """forced [1][L][K+1][k]: the GPU's routing; o: the oracle run with that
    routing forced (want_routing=True)."""
    if forced is None:
        return
    tol = TOL[cfg.wdtype]
    rl = o["router_logits"][0]
    L, K1, k = forced.shape[1:]
    for l in range(L):
        for j in range(K1):
            r = rl[l, j]
            gsel = [int(e) for e in forced[0, l, j]]
            assert len(set(gsel)) == k and min(gsel) >= 0 and max(gsel) < cfg.n_experts, (
                f"{label} layer {l} pos {j}: invalid routing {gsel}")
            own = [int(e) for e in oracle.topk(oracle.softmax(r), k)]
            stats["routings"] = stats.get("routings", 0) + 1
            if set(own) == set(gsel):
                continue
            band = tol * float(r.max() - r.min())
            kth = min(r[e] for e in own)
            worst = min(r[e] for e in gsel)
            stats["routing_near_ties"] = stats.get("routing_near_ties", 0) + 1
            assert worst >= kth - band, (
                f"{label} layer {l} pos {j}: GPU experts {sorted(gsel)} vs oracle {sorted(own)}, "
                f"logit gap {kth - worst:.4f} > band {band:.4f}")
