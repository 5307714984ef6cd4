"""Workload generators and the acceptance rule against figures the pages print."""
import json
import os

import numpy as np
import pytest
import torch

import workloads

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def _params(cfg):
    """(total, active per token) decoder parameters of a workload's model."""
    H, D = cfg.hidden, cfg.head_dim
    attn = cfg.qkv_dim * H + H * cfg.n_q * D
    exp = 3 * H * cfg.expert_inter
    per_layer = attn + cfg.n_experts * H + (cfg.n_experts + cfg.n_shared) * exp
    active_layer = attn + cfg.n_experts * H + (cfg.top_k + cfg.n_shared) * exp
    total = cfg.n_layers * per_layer + 2 * cfg.vocab * H
    active = cfg.n_layers * active_layer + cfg.vocab * H          # LM head, not the lookup
    return total, active


def test_twelve_layer_stack_matches_the_papers_decoder_size():
    g = GOLD["decoder_size"]
    cfg = workloads.get_config("moe_b32")
    total, active = _params(cfg)
    assert g["total_params_low"] <= total <= g["total_params_high"]
    assert abs(active - g["active_params"]) / g["active_params"] < 0.02
    assert (cfg.n_experts, cfg.n_shared, cfg.top_k) == (g["n_experts"], g["n_shared"], g["top_k"])


def test_page_context_of_batch1_workload():
    g = GOLD["page_context"]
    cfg = workloads.get_config("moe_b1")
    assert cfg.ctx == ("fixed", g["vision_tokens"] + g["text_tokens_per_page"])
    assert abs(g["output_tok_s"] / g["text_tokens_per_page"] - g["pages_per_s"]) < 0.01


def test_page_tau_follows_from_acceptance_rate(oracle_mod):
    """With acceptance rate r = accepted drafts / proposed drafts, the
    longest-prefix rule with a bonus token commits 1 + K r tokens per verify;
    the page's 57.6% and K = 3 give 2.728, printed as 2.7."""
    g = GOLD["tau_and_acceptance"]
    K, r = g["k_draft"], g["acceptance_rate"]
    assert round(1 + K * r, 1) == g["tokens_per_verify"]
    # independent per-position coins p with p + p^2 + p^3 = K r
    from scipy.optimize import brentq
    p = brentq(lambda x: x + x * x + x ** 3 - K * r, 0.0, 1.0)
    assert 0.74 < p < 0.76
    rng = np.random.default_rng(0)
    n = 40000
    coins = rng.random((n, K)) < p
    tau = 0.0
    acc = 0
    for i in range(n):
        gt = rng.integers(0, 1000, K + 1)
        d = np.where(coins[i], gt[:K], 1000 + np.arange(K))   # a non-match is never equal
        a, nxt = oracle_mod.accept(gt, d)
        assert nxt == gt[a]
        tau += a + 1
        acc += a
    tau /= n
    se = 1.0 / np.sqrt(n)
    assert abs(tau - (1 + K * r)) < 5 * se
    assert abs(acc / (n * K) - r) < 5 * se
    assert round(tau, 1) == g["tokens_per_verify"]


def _closed_form_mean_accepted(cfg):
    p = workloads.synth.match_probabilities(cfg).numpy()
    return float(np.mean(np.sum(np.cumprod(p, axis=1), axis=1)))


@pytest.mark.parametrize("name,expect", [("tiny_fp32", 1.176), ("moe_b1", 1.099),
                                         ("dense_fp8_b8", 3.600)])
def test_closed_form_accepted_lengths(name, expect):
    cfg = workloads.get_config(name)
    assert abs(_closed_form_mean_accepted(cfg) - expect) < 2e-3


def test_draft_stream_statistics_through_the_oracle(oracle_mod):
    """Drafts made by the workload's rule (copy the target's greedy token
    with the match probability, else a uniform token) give a mean accepted
    length equal to the closed form sum_n prod_{i<=n} p_i."""
    cfg = workloads.scaled(workloads.get_config("tiny_fp32"), hidden=64, n_q=2, n_kv=2,
                           head_dim=32, n_experts=4, expert_inter=32, vocab=256, steps=1200,
                           ctx=("fixed", 40), weight_std=0.2)
    w = workloads.make_weights(cfg)
    cap = workloads.capacity_for(cfg)
    k, v = workloads.kv_cache(cfg, capacity=cap)
    orc = oracle_mod.Oracle(cfg, w, cap)
    kc, vc = orc.kv_np(k, v)
    coins, rtok = workloads.draft_randomness(cfg)
    acc = []
    for s in range(cfg.steps):
        c0 = int(rtok[s, 0, 0])
        d = orc.make_drafts(kc, vc, 0, 40, c0, coins[s, 0], rtok[s, 0])
        out = orc.verify_step(kc, vc, [c0], d[None], [40])
        acc.append(int(out["accepted"][0]))
    acc = np.array(acc)
    mean = _closed_form_mean_accepted(cfg)
    assert abs(acc.mean() - mean) < 4 * acc.std() / np.sqrt(len(acc)) + 1e-3
    # the accepted length is never longer than the leading run of "match" coins
    lead = np.argmin(np.concatenate([coins[:, 0].numpy(), np.zeros((cfg.steps, 1), np.uint8)], 1),
                     axis=1)
    assert np.all(acc >= lead)


def test_generators_are_seeded_and_shaped():
    cfg = workloads.get_config("moe_b64_long")
    c1, c2 = workloads.context_lengths(cfg), workloads.context_lengths(cfg)
    assert torch.equal(c1, c2) and c1.min() >= 1000 and c1.max() <= 12000
    assert workloads.capacity_for(cfg) % 64 == 0
    assert workloads.capacity_for(cfg) >= 12000 + 100 * 4
    coins, toks = workloads.draft_randomness(workloads.get_config("moe_b32"))
    assert coins.shape == (1, 32, 3) and toks.max() < 129280
    p = workloads.synth.match_probabilities(workloads.get_config("moe_b32"))
    assert p.min() >= 0.4 and p.max() <= 0.8
