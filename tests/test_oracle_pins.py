"""Pins of the CPU oracle to things other than itself.

Each primitive is checked against a library routine with its own
implementation (torch, numpy, scipy), a closed form, or an invariant; the
whole step is checked against brute-force single-token greedy decoding (the
lossless property the pages state) and against a composition of torch library
operators.  All of these run on the CPU.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import workloads

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


# ------------------------------------------------------------------ formats
def test_e4m3_all_codes_match_torch(oracle_mod):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle_mod.e4m3_to_double(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9   # max finite, min subnormal


def test_bf16_widening_and_rounding_match_torch(oracle_mod):
    g = torch.Generator().manual_seed(1)
    bits = torch.randint(0, 1 << 16, (4000,), generator=g, dtype=torch.int32)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]          # drop inf / NaN patterns
    ref = bits.to(torch.int16).view(torch.bfloat16).double().numpy()
    got = np.array([oracle_mod.bf16_to_double(int(b) & 0xFFFF) for b in bits])
    assert np.array_equal(got, ref)
    # rounding: float32 inputs (torch rounds fp32 -> bf16 to nearest even)
    x = torch.randn(4000, generator=g, dtype=torch.float32) * 3
    ties = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 2 ** -130 * 1.5],
                        dtype=torch.float32)
    x = torch.cat([x, ties])
    ref = x.to(torch.bfloat16).double().numpy()
    got = np.array([oracle_mod.round_bf16(float(v)) for v in x])
    assert np.array_equal(got, ref)


# --------------------------------------------------------------- primitives
@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_matvec_matches_numpy_matmul(oracle_mod, dtype):
    g = torch.Generator().manual_seed(2)
    W = torch.randn(37, 53, generator=g) * 0.02
    x = np.random.default_rng(3).standard_normal(53)
    if dtype == "f32":
        Wd, scale, dense = W, None, W.double().numpy()
    elif dtype == "bf16":
        Wd, scale = W.to(torch.bfloat16), None
        dense = Wd.double().numpy()
    else:
        s = W.abs().amax(1, keepdim=True) / 448
        q = (W / s).to(torch.float8_e4m3fn)
        Wd, scale = q.view(torch.uint8), s.squeeze(1)
        dense = q.double().numpy() * s.double().numpy()
    got = oracle_mod.matvec(Wd, x, dtype, scale)
    np.testing.assert_allclose(got, dense @ x, rtol=1e-12, atol=1e-14)


def test_rmsnorm_matches_torch_and_invariants(oracle_mod):
    rng = np.random.default_rng(4)
    x = rng.standard_normal(96) * 3
    g = (1 + 0.1 * rng.standard_normal(96)).astype(np.float32)
    ref = F.rms_norm(torch.tensor(x), (96,), torch.tensor(g, dtype=torch.float64), eps=1e-6)
    np.testing.assert_allclose(oracle_mod.rmsnorm(x, g, 1e-6), ref.numpy(), rtol=1e-13)
    ones = np.ones(96, np.float32)
    y = oracle_mod.rmsnorm(x, ones, 0.0)
    assert abs(np.mean(y * y) - 1.0) < 1e-13                       # unit RMS
    np.testing.assert_allclose(oracle_mod.rmsnorm(7.5 * x, ones, 0.0), y, rtol=1e-13)
    c = np.full(96, -2.0)                                           # constant vector
    np.testing.assert_allclose(oracle_mod.rmsnorm(c, ones, 1e-6),
                               -1.0 / math.sqrt(1 + 1e-6 / 4.0), rtol=1e-14)


def test_rope_invariants(oracle_mod):
    D, theta = 64, 10000.0
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    np.testing.assert_array_equal(oracle_mod.rope(q, 0, theta), q)           # position 0
    for p in (1, 37, 4000):
        assert abs(np.linalg.norm(oracle_mod.rope(q, p, theta)) - np.linalg.norm(q)) < 1e-12
    # the score depends only on the relative offset
    s1 = oracle_mod.rope(q, 100, theta) @ oracle_mod.rope(k, 93, theta)
    s2 = oracle_mod.rope(q, 1007, theta) @ oracle_mod.rope(k, 1000, theta)
    assert abs(s1 - s2) < 1e-10
    # pairing (i, i + D/2) and the angle pos * theta^(-2i/D), turning e_i toward e_{i+D/2}
    for i in (0, 5, D // 2 - 1):
        e = np.zeros(D)
        e[i] = 1.0
        r = oracle_mod.rope(e, 3, theta)
        others = np.delete(r, [i, i + D // 2])
        assert np.all(others == 0)
        ang = math.atan2(r[i + D // 2], r[i])
        want = math.remainder(3 * theta ** (-2 * i / D), 2 * math.pi)
        assert abs(ang - want) < 1e-12


def test_rope_matches_complex_rotation(oracle_mod):
    """Rotate-half rotary is multiplication of (v_i + j v_{i+D/2}) by e^{j phi_i}."""
    D, theta, pos = 128, 10000.0, 1341
    v = np.random.default_rng(6).standard_normal(D)
    z = torch.complex(torch.tensor(v[: D // 2]), torch.tensor(v[D // 2:]))
    phi = pos * theta ** (-torch.arange(0, D // 2, dtype=torch.float64) * 2 / D)
    r = z * torch.polar(torch.ones_like(phi), phi)
    ref = np.concatenate([r.real.numpy(), r.imag.numpy()])
    np.testing.assert_allclose(oracle_mod.rope(v, pos, theta), ref, atol=1e-12)


def test_attention_special_cases_and_sdpa(oracle_mod):
    D = 64
    rng = np.random.default_rng(7)
    q = rng.standard_normal(D)
    v1 = rng.standard_normal((1, D)).astype(np.float32)
    k1 = rng.standard_normal((1, D)).astype(np.float32)
    np.testing.assert_allclose(oracle_mod.attend(q, k1, v1), v1[0], rtol=1e-15)   # one key
    K = np.repeat(k1, 9, 0)
    V = rng.standard_normal((9, D)).astype(np.float32)
    np.testing.assert_allclose(oracle_mod.attend(q, K, V), V.astype(np.float64).mean(0),
                               rtol=1e-12, atol=1e-14)                            # equal keys
    # scores ln 3 and 0 after the 1/sqrt(D) scale give weights 3/4 and 1/4
    qq = np.zeros(D)
    qq[0] = 1.0
    K2 = np.zeros((2, D), np.float32)
    K2[0, 0] = math.sqrt(D) * math.log(3.0)
    V2 = rng.standard_normal((2, D)).astype(np.float32)
    want = 0.75 * V2[0].astype(np.float64) + 0.25 * V2[1].astype(np.float64)
    np.testing.assert_allclose(oracle_mod.attend(qq, K2, V2), want, rtol=1e-6, atol=1e-7)
    # against torch's scaled_dot_product_attention
    Kr = rng.standard_normal((300, D)).astype(np.float32)
    Vr = rng.standard_normal((300, D)).astype(np.float32)
    ref = F.scaled_dot_product_attention(torch.tensor(q)[None, None],
                                         torch.tensor(Kr, dtype=torch.float64)[None],
                                         torch.tensor(Vr, dtype=torch.float64)[None])
    np.testing.assert_allclose(oracle_mod.attend(q, Kr, Vr), ref[0, 0].numpy(), rtol=1e-10,
                               atol=1e-12)


def test_softmax_topk_silu_against_libraries(oracle_mod):
    rng = np.random.default_rng(8)
    r = rng.standard_normal(64) * 0.7
    np.testing.assert_allclose(oracle_mod.softmax(r), scipy.special.softmax(r), rtol=1e-13)
    p = oracle_mod.softmax(r)
    got = oracle_mod.topk(p, 6)
    ref = np.argsort(-p.astype(np.float32), kind="stable")[:6]
    np.testing.assert_array_equal(got, ref)
    tie = np.array([0.1, 0.3, 0.3, 0.2, 0.3])
    np.testing.assert_array_equal(oracle_mod.topk(tie, 3), [1, 2, 4])   # lower index first
    for z in (-30.0, -1.5, 0.0, 0.7, 25.0):
        assert abs(oracle_mod.silu(z) - z * scipy.special.expit(z)) < 1e-15 * max(1, abs(z))


def test_argmax_and_acceptance_hand_cases(oracle_mod):
    lg = np.array([0.5, 2.0, -1.0, 2.0, 1.9])
    assert oracle_mod.argmax(lg) == int(np.argmax(lg)) == 1            # tie -> lowest index
    assert oracle_mod.argmax(np.array([1.0, np.nan, 0.0])) == -1
    # ties are decided in fp32: these differ in fp64 but not after rounding
    assert oracle_mod.argmax(np.array([1.0, 1.0 + 1e-12])) == 0
    K = 3
    g = [11, 12, 13, 14]
    assert oracle_mod.accept(g, [11, 12, 13]) == (3, 14)               # all accepted: bonus g_K
    assert oracle_mod.accept(g, [99, 12, 13]) == (0, 11)               # first rejected
    assert oracle_mod.accept(g, [11, 99, 13]) == (1, 12)               # rejected at 2
    assert oracle_mod.accept(g, [11, 12, 99]) == (2, 13)               # rejected at 3
    assert oracle_mod.accept(g, [11, 99, 99]) == (1, 12)
    assert K == 3


# --------------------------------------------------------------------- MoE
def _small_moe(**kw):
    base = workloads.scaled(workloads.get_config("tiny_fp32"), hidden=64, n_q=2, n_kv=2,
                            head_dim=32, n_experts=6, expert_inter=48, top_k=2, n_shared=1,
                            vocab=300, norm_gain_std=0.1, weight_std=0.15)
    return workloads.scaled(base, **kw)


def test_moe_single_expert_reduces_to_dense_swiglu(oracle_mod):
    cfg = _small_moe(n_experts=1, top_k=1, n_shared=0)
    w = workloads.make_weights(cfg)
    orc = oracle_mod.Oracle(cfg, w, 64)
    h = np.random.default_rng(9).standard_normal(cfg.hidden)
    y, sel = oracle_mod.ffn(orc, 0, h)
    L = w["layers"][0]
    gu = L["w_gate_up"][0].double()
    I = cfg.expert_inter
    ht = torch.tensor(h)
    ref = (F.silu(gu[:I] @ ht) * (gu[I:] @ ht)) @ L["w_down"][0].double().T
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-14)
    assert sel[0] == 0


@pytest.mark.parametrize("renorm", [0, 1])
def test_moe_equals_masked_dense_evaluation(oracle_mod, renorm):
    cfg = _small_moe(renorm_topk=renorm)
    w = workloads.make_weights(cfg)
    orc = oracle_mod.Oracle(cfg, w, 64)
    L = w["layers"][0]
    I = cfg.expert_inter
    for seed in range(5):
        h = torch.tensor(np.random.default_rng(10 + seed).standard_normal(cfg.hidden))
        y, sel = oracle_mod.ffn(orc, 0, h.numpy())
        p = torch.softmax(L["w_router"].double() @ h, 0)
        top = torch.topk(p.float(), cfg.top_k).indices
        gate = torch.zeros_like(p)
        gate[top] = p[top] / (p[top].sum() if renorm else 1.0)
        ref = torch.zeros_like(h)
        for e in range(cfg.n_experts):                       # every expert, masked
            gu = L["w_gate_up"][e].double()
            ye = (F.silu(gu[:I] @ h) * (gu[I:] @ h)) @ L["w_down"][e].double().T
            ref += gate[e] * ye
        for s in range(cfg.n_shared):
            gu = L["w_sh_gate_up"][s].double()
            ref += (F.silu(gu[:I] @ h) * (gu[I:] @ h)) @ L["w_sh_down"][s].double().T
        np.testing.assert_allclose(y, ref.numpy(), rtol=1e-11, atol=1e-13)
        assert set(sel.tolist()) == set(top.tolist())


# -------------------------------------------------------------- whole step
def _torch_reference_logits(cfg, w, kc, vc, ctx, tokens):
    """The verify forward composed from torch library operators in float64:
    rms_norm, linear, complex rotation, scaled_dot_product_attention with a
    causal mask, softmax / topk routing, silu."""
    H, D, nq, nkv = cfg.hidden, cfg.head_dim, cfg.n_q, cfg.n_kv
    n = len(tokens)
    kcache = torch.tensor(kc[0]).double()
    vcache = torch.tensor(vc[0]).double()
    x = w["embed"].double()[torch.tensor(tokens)]
    pos = ctx + torch.arange(n, dtype=torch.float64)
    inv = cfg.rope_theta ** (-torch.arange(0, D // 2, dtype=torch.float64) * 2 / D)
    rot = torch.polar(torch.ones(n, D // 2, dtype=torch.float64), pos[:, None] * inv[None])

    def rope(t):   # t [n, heads, D]
        z = torch.complex(t[..., : D // 2], t[..., D // 2:]) * rot[:, None, :]
        return torch.cat([z.real, z.imag], -1)

    for l, L in enumerate(w["layers"]):
        h = F.rms_norm(x, (H,), L["attn_norm"].double(), eps=cfg.rms_eps)
        qkv = F.linear(h, L["w_qkv"].double())
        q = rope(qkv[:, : nq * D].reshape(n, nq, D))
        k = rope(qkv[:, nq * D:(nq + nkv) * D].reshape(n, nkv, D))
        v = qkv[:, (nq + nkv) * D:].reshape(n, nkv, D)
        kcache[l, :, ctx:ctx + n] = k.float().double().transpose(0, 1)   # fp32 cache
        vcache[l, :, ctx:ctx + n] = v.float().double().transpose(0, 1)
        keys = kcache[l, :, : ctx + n]
        vals = vcache[l, :, : ctx + n]
        rep = nq // nkv
        keys = keys.repeat_interleave(rep, 0)
        vals = vals.repeat_interleave(rep, 0)
        mask = torch.arange(ctx + n)[None, :] <= (ctx + torch.arange(n))[:, None]
        o = F.scaled_dot_product_attention(q.transpose(0, 1), keys, vals, attn_mask=mask)
        x = x + F.linear(o.transpose(0, 1).reshape(n, nq * D), L["w_o"].double())
        h = F.rms_norm(x, (H,), L["ffn_norm"].double(), eps=cfg.rms_eps)
        p = torch.softmax(F.linear(h, L["w_router"].double()), -1)
        top = torch.topk(p.float(), cfg.top_k, dim=-1).indices
        I = cfg.expert_inter
        y = torch.zeros_like(x)
        for j in range(n):
            for e in top[j].tolist():
                gu = L["w_gate_up"][e].double()
                y[j] += p[j, e] * F.linear(F.silu(gu[:I] @ h[j]) * (gu[I:] @ h[j]),
                                           L["w_down"][e].double())
            for s in range(cfg.n_shared):
                gu = L["w_sh_gate_up"][s].double()
                y[j] += F.linear(F.silu(gu[:I] @ h[j]) * (gu[I:] @ h[j]),
                                 L["w_sh_down"][s].double())
        x = x + y
    f = F.rms_norm(x, (H,), w["final_norm"].double(), eps=cfg.rms_eps)
    return F.linear(f, w["lm_head"].double()).numpy(), x.numpy()


def test_step_matches_torch_operator_composition(oracle_mod):
    cfg = workloads.scaled(workloads.get_config("tiny_fp32"), norm_gain_std=0.1, n_layers=2,
                           n_q=4, n_kv=2)
    w = workloads.make_weights(cfg)
    cap = workloads.capacity_for(cfg)
    k, v = workloads.kv_cache(cfg, capacity=cap)
    orc = oracle_mod.Oracle(cfg, w, cap)
    kc, vc = orc.kv_np(k, v)
    k0, v0 = kc.copy(), vc.copy()
    ctx = 200
    tokens = [5, 900, 17, 333]
    out = orc.verify_step(kc, vc, [tokens[0]], [tokens[1:]], [ctx], want_logits=True,
                          want_hidden=True)
    ref_logits, ref_x = _torch_reference_logits(cfg, w, k0, v0, ctx, tokens)
    np.testing.assert_allclose(out["logits"][0], ref_logits, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(out["hidden"][0], ref_x, rtol=1e-9, atol=1e-11)
    np.testing.assert_array_equal(out["target"][0], np.argmax(ref_logits.astype(np.float32), -1))


def _lossless_case(oracle_mod, cfg, seed_steps=3):
    """Verify-step output equals plain greedy decoding, and its per-position
    logits equal those of K+1 chained single-token decodes bit for bit."""
    w = workloads.make_weights(cfg)
    cap = workloads.capacity_for(cfg)
    k, v = workloads.kv_cache(cfg, capacity=cap)
    orc = oracle_mod.Oracle(cfg, w, cap)
    ctx = workloads.context_lengths(cfg)
    com = workloads.committed_tokens(cfg)
    coins, rtok = workloads.draft_randomness(cfg, steps=seed_steps)
    K = cfg.k_draft
    seen_accept = set()
    for s in range(seed_steps):
        for b in range(cfg.batch):
            kc, vc = orc.kv_np(k[b:b + 1], v[b:b + 1])
            c0, t0 = int(ctx[b]), int(com[b])
            drafts = orc.make_drafts(kc, vc, 0, c0, t0, coins[s, b], rtok[s, b])
            out = orc.verify_step(kc, vc, [t0], drafts[None], [c0], want_logits=True)
            a, nxt = int(out["accepted"][0]), int(out["next_tok"][0])
            seen_accept.add(a)
            # teacher-forced single-token decodes over the same block
            kc2, vc2 = orc.kv_np(k[b:b + 1], v[b:b + 1])
            block = [t0] + drafts.tolist()
            for j in range(K + 1):
                g, lg, _ = orc.decode_one(kc2, vc2, 0, c0 + j, block[j], want_logits=True)
                assert g == out["target"][0, j]
                np.testing.assert_array_equal(lg, out["logits"][0, j])
            np.testing.assert_array_equal(kc2, kc)
            np.testing.assert_array_equal(vc2, vc)
            # plain greedy autoregressive decoding from the committed token
            kc3, vc3 = orc.kv_np(k[b:b + 1], v[b:b + 1])
            ar, prev = [], t0
            for j in range(a + 1):
                prev, _, _ = orc.decode_one(kc3, vc3, 0, c0 + j, prev)
                ar.append(prev)
            assert drafts[:a].tolist() == ar[:a] and nxt == ar[a]
            assert out["ctx_out"][0] == c0 + a + 1
    return seen_accept


def test_lossless_tiny(oracle_mod):
    cfg = workloads.scaled(workloads.get_config("tiny_fp32"), batch=4, n_layers=2)
    seen = _lossless_case(oracle_mod, cfg)
    assert len(seen) >= 2


def test_lossless_moe_bf16_scaled(oracle_mod):
    cfg = workloads.scaled(workloads.get_config("moe_b1"), hidden=128, n_q=2, n_kv=2,
                           head_dim=64, n_experts=8, expert_inter=64, top_k=3, n_shared=2,
                           vocab=512, n_layers=2, batch=3, ctx=("uniform", 20, 90),
                           draft_p=("const", 0.8))
    _lossless_case(oracle_mod, cfg)


def test_lossless_dense_fp8_gqa_scaled(oracle_mod):
    cfg = workloads.scaled(workloads.get_config("dense_fp8_b8"), hidden=128, n_q=4, n_kv=2,
                           head_dim=32, dense_inter=192, vocab=400, n_layers=2, batch=2,
                           k_draft=7, ctx=("uniform", 30, 80))
    _lossless_case(oracle_mod, cfg, seed_steps=2)


def test_error_status(oracle_mod):
    cfg = workloads.get_config("tiny_fp32")
    w = workloads.make_weights(cfg)
    cap = workloads.capacity_for(cfg)
    k, v = workloads.kv_cache(cfg, capacity=cap)
    orc = oracle_mod.Oracle(cfg, w, cap)
    kc, vc = orc.kv_np(k, v)
    out = orc.verify_step(kc, vc, [cfg.vocab], [[1, 2, 3]], [10])
    assert out["status"][0] == oracle_mod.BAD_TOKEN and out["accepted"][0] == -1
    assert out["ctx_out"][0] == 10
    out = orc.verify_step(kc, vc, [1], [[1, 2, 3]], [cap - 3])
    assert out["status"][0] == oracle_mod.CAPACITY and out["next_tok"][0] == -1


def test_routing_hook_forcing_own_choice_is_identity(oracle_mod):
    """Forcing the oracle's own expert choice reproduces the free run bit for
    bit; forcing another choice changes the result; the reported router logits
    give back the reported selection through softmax + top-k."""
    cfg = workloads.scaled(_small_moe(), n_layers=2, batch=1, k_draft=3)
    w = workloads.make_weights(cfg)
    cap = 128
    k, v = workloads.kv_cache(cfg, capacity=cap)
    orc = oracle_mod.Oracle(cfg, w, cap)
    args = ([3], [[10, 20, 30]], [50])
    kc, vc = orc.kv_np(k, v)
    free = orc.verify_step(kc, vc, *args, want_logits=True, want_routing=True)
    kc, vc = orc.kv_np(k, v)
    same = orc.verify_step(kc, vc, *args, want_logits=True, force_sel=free["sel"])
    np.testing.assert_array_equal(same["logits"], free["logits"])
    for l in range(cfg.n_layers):
        for j in range(4):
            r = free["router_logits"][0, l, j]
            np.testing.assert_array_equal(free["sel"][0, l, j],
                                          oracle_mod.topk(oracle_mod.softmax(r), cfg.top_k))
    other = free["sel"].copy()
    other[0, 0, 0] = [e for e in range(cfg.n_experts) if e not in other[0, 0, 0]][:cfg.top_k]
    kc, vc = orc.kv_np(k, v)
    diff = orc.verify_step(kc, vc, *args, want_logits=True, force_sel=other)
    assert np.abs(diff["logits"] - free["logits"]).max() > 1e-6


# ------------------------------------------------------------------ MXFP4
# OCP Microscaling Formats (MX) v1.0, E2M1 element encoding: the 16 codes
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
              -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e2m1_and_e8m0_codes(oracle_mod):
    got = [oracle_mod.e2m1_to_double(c) for c in range(16)]
    assert got == E2M1_TABLE
    assert np.signbit(got[8])
    assert oracle_mod.e8m0_to_double(127) == 1.0
    assert oracle_mod.e8m0_to_double(0) == 2.0 ** -127
    assert oracle_mod.e8m0_to_double(254) == 2.0 ** 127
    assert math.isnan(oracle_mod.e8m0_to_double(255))


def _mx_dequant_numpy(packed, scales):
    """Reference decoding written from the format's definition: element 2i in
    the low nibble of byte i, value = table[code] * 2^(scale - 127)."""
    lo, hi = packed & 15, packed >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(packed.shape[0], -1)
    vals = np.array(E2M1_TABLE)[codes]
    return vals * np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)


def test_mxfp4_matvec_matches_numpy(oracle_mod):
    rng = np.random.default_rng(4)
    N, K = 37, 256
    packed = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = rng.integers(110, 140, (N, K // 32), dtype=np.uint8)
    x = rng.normal(size=K)
    y = oracle_mod.matvec(packed, x, dtype="mxfp4", scale=scales)
    np.testing.assert_allclose(y, _mx_dequant_numpy(packed, scales) @ x, rtol=1e-12, atol=1e-12)


def test_mxfp4_quantizer_rounds_to_nearest(oracle_mod):
    """The workloads' MXFP4 quantizer: block scale 2^(floor(log2 amax) - 2),
    every element the nearest representable value (brute force over the 16
    codes), ties to the even code."""
    from workloads.synth import _quant_mxfp4
    g = torch.Generator().manual_seed(9)
    w = torch.randn(24, 128, generator=g) * 0.02
    w[3, 5] = 0.0
    w[4, :32] = 0.0                        # an all-zero block
    packed, scales = _quant_mxfp4(w)
    deq = _mx_dequant_numpy(packed.numpy(), scales.numpy())
    wn = w.double().numpy()
    for r in range(24):
        for blk in range(4):
            seg = wn[r, 32 * blk:32 * blk + 32]
            amax = np.abs(seg).max()
            e = int(np.floor(np.log2(amax))) - 2 if amax > 0 else -127
            assert int(scales[r, blk]) == e + 127
            cand = np.array(E2M1_TABLE) * 2.0 ** e
            for i, v in enumerate(seg):
                best = np.abs(cand - v).min()
                assert abs(deq[r, 32 * blk + i] - v) == best
    # ties go to the even code: 2.5 -> 2, 5 -> 4, 0.25 -> 0 (block amax 5 -> scale 1)
    t = torch.zeros(1, 32)
    t[0, :4] = torch.tensor([4.0, 2.5, 5.0, 0.25])
    p2, s2 = _quant_mxfp4(t)
    d2 = _mx_dequant_numpy(p2.numpy(), s2.numpy())[0, :4]
    assert d2.tolist() == [4.0, 2.0, 4.0, 0.0]


def test_lossless_moe_mxfp4_scaled(oracle_mod):
    cfg = workloads.scaled(workloads.get_config("moe_b1_mxfp4"), hidden=128, n_q=2, n_kv=2,
                           head_dim=64, n_experts=8, expert_inter=64, top_k=3, n_shared=2,
                           vocab=512, n_layers=2, batch=3, ctx=("uniform", 20, 90),
                           draft_p=("const", 0.8))
    _lossless_case(oracle_mod, cfg)


# ------------------------------------------------------------------ FastMTP
def _torch_dense_block(cfg, L, x, kcache, vcache, ctx):
    """One dense pre-norm decoder layer on residual rows x [n][H] at positions
    ctx .. ctx+n-1 composed from torch operators (float64; the caches
    [n_kv][cap][D] are written in place, rounded to fp32)."""
    H, D, nq, nkv = cfg.hidden, cfg.head_dim, cfg.n_q, cfg.n_kv
    n = x.shape[0]
    pos = ctx + torch.arange(n, dtype=torch.float64)
    inv = cfg.rope_theta ** (-torch.arange(0, D // 2, dtype=torch.float64) * 2 / D)
    rot = torch.polar(torch.ones(n, D // 2, dtype=torch.float64), pos[:, None] * inv[None])

    def rope(t):
        z = torch.complex(t[..., : D // 2], t[..., D // 2:]) * rot[:, None, :]
        return torch.cat([z.real, z.imag], -1)

    h = F.rms_norm(x, (H,), L["attn_norm"].double(), eps=cfg.rms_eps)
    qkv = F.linear(h, L["w_qkv"].double())
    q = rope(qkv[:, : nq * D].reshape(n, nq, D))
    k = rope(qkv[:, nq * D:(nq + nkv) * D].reshape(n, nkv, D))
    v = qkv[:, (nq + nkv) * D:].reshape(n, nkv, D)
    kcache[:, ctx:ctx + n] = k.float().double().transpose(0, 1)
    vcache[:, ctx:ctx + n] = v.float().double().transpose(0, 1)
    keys = kcache[:, : ctx + n].repeat_interleave(nq // nkv, 0)
    vals = vcache[:, : ctx + n].repeat_interleave(nq // nkv, 0)
    mask = torch.arange(ctx + n)[None, :] <= (ctx + torch.arange(n))[:, None]
    o = F.scaled_dot_product_attention(q.transpose(0, 1), keys, vals, attn_mask=mask)
    x = x + F.linear(o.transpose(0, 1).reshape(n, nq * D), L["w_o"].double())
    h = F.rms_norm(x, (H,), L["ffn_norm"].double(), eps=cfg.rms_eps)
    I = cfg.dense_inter
    gu = L["w_gate_up"].double()
    return x + F.linear(F.silu(F.linear(h, gu[:I])) * F.linear(h, gu[I:]), L["w_down"].double())


@pytest.mark.parametrize("accepted", [0, 2, 3])
def test_mtp_draft_matches_torch_composition(oracle_mod, accepted):
    """FastMTP drafting (Jina-OCR-v1 paper, section 3.1) against the same
    recursion composed from torch operators: z = P [N_e(e); N_h(a)], u =
    N_o(B(z)), draft = argmax W_lm u, depth 1 over the committed rows, deeper
    depths on the previous depth's u and draft."""
    base = workloads.scaled(workloads.get_config("tiny_fp32"), n_q=4, n_kv=2, norm_gain_std=0.1)
    mc = workloads.mtp_config(base)
    tw = workloads.make_weights(base)
    mw = workloads.mtp_weights(base)
    cap = workloads.capacity_for(base) + 16
    k, v = workloads.kv_cache(mc, capacity=cap)
    orc = oracle_mod.Oracle(mc, workloads.mtp_model_weights(tw, mw), cap)
    kc, vc = orc.kv_np(k, v)
    kt, vt = torch.tensor(kc[0, 0]).double(), torch.tensor(vc[0, 0]).double()
    K, H, ctx = base.k_draft, base.hidden, 200
    g = torch.Generator().manual_seed(accepted)
    drafts = torch.randint(0, base.vocab, (K,), generator=g).tolist()
    nxt = 77
    bstate = torch.randn(accepted + 1, H, generator=g, dtype=torch.float64)
    got, gaps = orc.mtp_draft(mw, kc, vc, 0, ctx, accepted, drafts, nxt, bstate.numpy())

    def zrows(toks, states):
        e = F.rms_norm(tw["embed"].double()[torch.tensor(toks)], (H,), mw["enorm"].double(),
                       eps=base.rms_eps)
        s = F.rms_norm(states, (H,), mw["hnorm"].double(), eps=base.rms_eps)
        return F.linear(torch.cat([e, s], -1), mw["eh_proj"].double())

    def head(xo):
        f = F.rms_norm(xo, (H,), tw["final_norm"].double(), eps=base.rms_eps)
        return f, F.linear(f, tw["lm_head"].double())

    toks = [drafts[j] if j < accepted else nxt for j in range(accepted + 1)]
    xo = _torch_dense_block(mc, mw["block"], zrows(toks, bstate), kt, vt, ctx)
    f, lg = head(xo)
    want = [int(torch.argmax(lg[accepted].float()))]
    u = f[accepted:accepted + 1]
    for k_ in range(2, K + 1):
        xo = _torch_dense_block(mc, mw["block"], zrows([want[-1]], u), kt, vt, ctx + accepted + k_ - 1)
        f, lg = head(xo)
        want.append(int(torch.argmax(lg[0].float())))
        u = f
    assert got.tolist() == want
    assert np.all(gaps > 0)
    # the block's cache now holds the committed rows and the deeper depths' rows
    np.testing.assert_allclose(kc[0, 0, :, : ctx + accepted + K], kt[:, : ctx + accepted + K].numpy(),
                               rtol=1e-6, atol=1e-9)
