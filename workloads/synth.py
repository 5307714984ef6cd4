"""Seeded synthetic inputs: weights, KV cache, context lengths, draft randomness.

Every tensor has its own seed, derived from the workload seed and the tensor's
name, so any one of them can be regenerated alone.  Generation uses torch on
the requested device; values drawn on different devices differ, so a test that
feeds both the GPU library and the CPU oracle draws once and copies.

Distributions (the pages train real weights; these stand in for them):
  * every linear weight and the embedding: N(0, 0.02^2); norm gains 1
    (or 1 + N(0, norm_gain_std^2) for tests that need distinct gains);
  * bf16 storage: fp32 samples rounded to nearest-even bf16;
  * fp8 storage: one scale per output row, s = max|w| / 448, codes
    e4m3fn(round-to-nearest-even(w / s)), clamped to +-448;
  * cached keys/values before the step: N(0, (0.02 sqrt(H))^2), the spread a
    unit-RMS input gives through an N(0, 0.02^2) projection, in cache storage;
  * context lengths: fixed, uniform integer, or log-uniform (rounded);
  * drafts: per position a Bernoulli coin with the workload's match
    probability and a uniform token used when the coin says "no match".
"""
from __future__ import annotations

import math
import zlib

import torch

from .configs import VerifyConfig

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def tensor_seed(base: int, name: str) -> int:
    return (zlib.crc32(name.encode()) ^ (base * 0x9E3779B1)) & 0x7FFFFFFF


def _gen(device, base: int, name: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(tensor_seed(base, name))
    return g


def _normal(shape, std, device, base, name) -> torch.Tensor:
    g = _gen(device, base, name)
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32) * std


def _quant_e4m3_rows(w: torch.Tensor):
    """Per-output-row e4m3fn codes (uint8) and fp32 scales."""
    s = w.abs().amax(dim=-1, keepdim=True) / 448.0
    s = torch.where(s > 0, s, torch.ones_like(s))
    q = (w / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), s.squeeze(-1).to(torch.float32)


# E2M1 magnitudes by code (OCP Microscaling formats v1.0: 1 sign, 2 exponent
# bits with bias 1, 1 mantissa bit)
_E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _quant_mxfp4(w: torch.Tensor):
    """MXFP4 along the last dimension (a multiple of 32): per 32-element block
    an E8M0 scale 2^e with e = floor(log2(amax)) - 2 (the largest E2M1
    exponent), elements w / 2^e rounded to the nearest E2M1 value (ties to the
    even code) and saturated at +-6.  Returns (codes packed two per byte, even
    element in the low 4 bits, uint8 [..., K/2]; scale bytes e + 127, uint8
    [..., K/32])."""
    shp = w.shape
    K = shp[-1]
    wb = w.to(torch.float64).reshape(*shp[:-1], K // 32, 32)
    amax = wb.abs().amax(dim=-1, keepdim=True)
    e = torch.where(amax > 0, torch.floor(torch.log2(torch.where(amax > 0, amax, 1.0))) - 2,
                    torch.full_like(amax, -127.0)).clamp(-127, 127)
    x = (wb / torch.exp2(e)).abs()
    grid = torch.tensor(_E2M1, dtype=torch.float64, device=w.device)
    d = (x.unsqueeze(-1) - grid).abs()
    odd = torch.tensor([0, 1, 0, 1, 0, 1, 0, 1], dtype=torch.float64, device=w.device)
    code = torch.argmin(d + odd * 1e-9 * (d.amin(-1, keepdim=True) == d), dim=-1)
    code = code.to(torch.uint8) | ((wb < 0).to(torch.uint8) << 3)
    code = code.reshape(*shp[:-1], K)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return packed.contiguous(), (e.squeeze(-1) + 127).to(torch.uint8).contiguous()


def _linear(cfg: VerifyConfig, shape, device, name, mx_ok=False):
    """A linear weight of the given shape in the workload's storage format
    (the workload's `mx` format for the weight-streaming matrices when it
    names one).  Returns (tensor, per-row scale, block scales or None)."""
    w = _normal(shape, cfg.weight_std, device, cfg.seed, name)
    if mx_ok and cfg.mx == "mxfp4":
        return _quant_mxfp4(w)
    if cfg.wdtype == "fp8":
        return _quant_e4m3_rows(w)
    return w.to(_TORCH_DT[cfg.wdtype]), None


def _gain(cfg: VerifyConfig, n, device, name):
    if cfg.norm_gain_std == 0.0:
        return torch.ones(n, dtype=torch.float32, device=device)
    return 1.0 + _normal((n,), cfg.norm_gain_std, device, cfg.seed, name)


def make_weights(cfg: VerifyConfig, device="cpu") -> dict:
    """All weights of the target decoder, row-major [out][in] per matrix.

    Keys: embed [V][H]; final_norm [H]; lm_head [V][H] (+ lm_scale [V] for
    fp8); layers: list of dicts with attn_norm [H], w_qkv [(n_q+2n_kv)D][H],
    w_o [H][n_q D], ffn_norm [H] and either (MoE) w_router [E][H],
    w_gate_up [E][2I][H], w_down [E][H][I], w_sh_gate_up [S][2I][H],
    w_sh_down [S][H][I], or (dense) w_gate_up [2I][H], w_down [H][I].  Each
    matrix `w_x` stored in fp8 has a companion `s_x` of per-row scales.  With
    mx = "mxfp4" the expert matrices and the LM head are MXFP4: `w_x` holds
    the packed codes [..][K/2] (uint8) and `s_x` (lm_scale) the E8M0 block
    scales [..][K/32] (uint8).
    """
    H, D = cfg.hidden, cfg.head_dim
    out = {}
    emb = _normal((cfg.vocab, H), cfg.weight_std, device, cfg.seed, "embed")
    out["embed"] = emb.to(_TORCH_DT[cfg.embdtype])
    del emb
    layers = []
    for l in range(cfg.n_layers):
        p = f"layer{l}."
        L = {"attn_norm": _gain(cfg, H, device, p + "attn_norm"),
             "ffn_norm": _gain(cfg, H, device, p + "ffn_norm")}
        L["w_qkv"], L["s_qkv"] = _linear(cfg, (cfg.qkv_dim, H), device, p + "w_qkv")
        L["w_o"], L["s_o"] = _linear(cfg, (H, cfg.n_q * D), device, p + "w_o")
        if cfg.ffn == "moe":
            E, I, S = cfg.n_experts, cfg.expert_inter, cfg.n_shared
            L["w_router"], L["s_router"] = _linear(cfg, (E, H), device, p + "w_router")
            L["w_gate_up"], L["s_gate_up"] = _linear(cfg, (E, 2 * I, H), device, p + "w_gate_up",
                                                    mx_ok=True)
            L["w_down"], L["s_down"] = _linear(cfg, (E, H, I), device, p + "w_down", mx_ok=True)
            L["w_sh_gate_up"], L["s_sh_gate_up"] = _linear(cfg, (S, 2 * I, H), device,
                                                          p + "w_sh_gate_up", mx_ok=True)
            L["w_sh_down"], L["s_sh_down"] = _linear(cfg, (S, H, I), device, p + "w_sh_down",
                                                    mx_ok=True)
        else:
            I = cfg.dense_inter
            L["w_gate_up"], L["s_gate_up"] = _linear(cfg, (2 * I, H), device, p + "w_gate_up")
            L["w_down"], L["s_down"] = _linear(cfg, (H, I), device, p + "w_down")
        layers.append(L)
    out["layers"] = layers
    out["final_norm"] = _gain(cfg, H, device, "final_norm")
    out["lm_head"], out["lm_scale"] = _linear(cfg, (cfg.vocab, H), device, "lm_head",
                                              mx_ok=True)
    return out


def capacity_for(cfg: VerifyConfig) -> int:
    """Cache slots per (sequence, layer, KV head): the largest starting
    context plus every position the workload's steps can add, rounded up to a
    multiple of 64."""
    kind = cfg.ctx[0]
    hi = cfg.ctx[1] if kind == "fixed" else cfg.ctx[2]
    need = hi + cfg.steps * (cfg.k_draft + 1)
    return (need + 63) // 64 * 64


def context_lengths(cfg: VerifyConfig) -> torch.Tensor:
    """Starting context length of every sequence (int32, CPU)."""
    g = _gen("cpu", cfg.seed, "ctx_lens")
    B = cfg.batch
    kind = cfg.ctx[0]
    if kind == "fixed":
        return torch.full((B,), cfg.ctx[1], dtype=torch.int32)
    if kind == "uniform":
        lo, hi = cfg.ctx[1], cfg.ctx[2]
        return torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    if kind == "loguniform":
        lo, hi = cfg.ctx[1], cfg.ctx[2]
        u = torch.rand(B, generator=g, dtype=torch.float64)
        v = torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
        return torch.round(v).clamp(lo, hi).to(torch.int32)
    raise ValueError(kind)


def committed_tokens(cfg: VerifyConfig) -> torch.Tensor:
    """The last committed token of every sequence (int32, CPU)."""
    g = _gen("cpu", cfg.seed, "committed")
    return torch.randint(0, cfg.vocab, (cfg.batch,), generator=g, dtype=torch.int64).to(torch.int32)


def match_probabilities(cfg: VerifyConfig) -> torch.Tensor:
    """Per-(sequence, draft position) probability that the draft equals the
    target's greedy token, float64 [B][K]."""
    B, K = cfg.batch, cfg.k_draft
    kind = cfg.draft_p[0]
    if kind == "const":
        return torch.full((B, K), float(cfg.draft_p[1]), dtype=torch.float64)
    if kind == "per_seq_uniform":
        g = _gen("cpu", cfg.seed, "draft_p_seq")
        lo, hi = cfg.draft_p[1], cfg.draft_p[2]
        p = lo + (hi - lo) * torch.rand(B, 1, generator=g, dtype=torch.float64)
        return p.expand(B, K).clone()
    if kind == "decay":
        p0, r = cfg.draft_p[1], cfg.draft_p[2]
        p = torch.tensor([p0 * r ** i for i in range(K)], dtype=torch.float64)
        return p.expand(B, K).clone()
    raise ValueError(kind)


def draft_randomness(cfg: VerifyConfig, steps: int | None = None):
    """Coins (uint8 [S][B][K]: 1 = the draft copies the target's greedy token)
    and fallback tokens (int32 [S][B][K], uniform over the vocabulary)."""
    S = cfg.steps if steps is None else steps
    B, K = cfg.batch, cfg.k_draft
    p = match_probabilities(cfg)
    g = _gen("cpu", cfg.seed, "draft_coins")
    u = torch.rand(S, B, K, generator=g, dtype=torch.float64)
    coins = (u < p.unsqueeze(0)).to(torch.uint8)
    g2 = _gen("cpu", cfg.seed, "draft_tokens")
    toks = torch.randint(0, cfg.vocab, (S, B, K), generator=g2, dtype=torch.int64).to(torch.int32)
    return coins, toks


def kv_cache(cfg: VerifyConfig, device="cpu", capacity: int | None = None):
    """Key and value caches before the step, natural layout
    [B][L][n_kv][capacity][D] in the cache storage type."""
    cap = capacity_for(cfg) if capacity is None else capacity
    shape = (cfg.batch, cfg.n_layers, cfg.n_kv, cap, cfg.head_dim)
    std = cfg.weight_std * math.sqrt(cfg.hidden)
    dt = _TORCH_DT[cfg.kvdtype]
    out = []
    for name in ("k_cache", "v_cache"):
        t = torch.empty(shape, dtype=dt, device=device)
        for b in range(cfg.batch):   # per sequence keeps the fp32 temporary small
            t[b] = _normal(shape[1:], std, device, cfg.seed, f"{name}.{b}").to(dt)
        out.append(t)
    return out[0], out[1]


def sampled_drafts(cfg: VerifyConfig, batch: int | None = None, step: int = 0,
                   sigma: float | None = None):
    """Inputs of a sampled (rejection-sampling) verify step, on the CPU:
    draft distributions q [B][K][V] (fp32; each row the normalised weights
    exp(sigma * N(0, 1)), the spread of the target's own logits by default:
    sigma = weight_std * sqrt(hidden)), drafts [B][K] (int32, drawn from q),
    acceptance uniforms u [B][K] (fp32 in [0, 1)), and the generator seed and
    offset of the step's Gumbel noise."""
    B = cfg.batch if batch is None else batch
    K, V = cfg.k_draft, cfg.vocab
    sig = cfg.weight_std * math.sqrt(cfg.hidden) if sigma is None else sigma
    g = _gen("cpu", cfg.seed, f"draft_dist.{step}")
    w = torch.exp(sig * torch.randn(B, K, V, generator=g, dtype=torch.float64))
    q = w / w.sum(-1, keepdim=True)
    g2 = _gen("cpu", cfg.seed, f"draft_pick.{step}")
    drafts = torch.multinomial(q.reshape(B * K, V), 1, generator=g2).reshape(B, K).to(torch.int32)
    g3 = _gen("cpu", cfg.seed, f"accept_u.{step}")
    u = torch.rand(B, K, generator=g3, dtype=torch.float32)
    seed = tensor_seed(cfg.seed, "gumbel_seed") * 0x100000001 & (2 ** 64 - 1)
    return {"q": q.to(torch.float32), "drafts": drafts, "u": u, "seed": seed, "offset": step}


def mtp_weights(cfg: VerifyConfig, device="cpu") -> dict:
    """The FastMTP draft head of a target workload (Jina-OCR-v1 paper,
    section 3.1; the released checkpoint names enorm, hnorm, eh_proj and
    mtp_block): RMSNorm gains enorm and hnorm [H] (1, or 1 + N(0,
    norm_gain_std^2)), the projection eh_proj [H][2H] (+ s_eh_proj for fp8)
    and one dense decoder layer `block` (attn_norm, w_qkv, w_o, ffn_norm,
    w_gate_up [2 I_d][H], w_down [H][I_d]) with I_d = cfg.dense_inter if set,
    else 4 H.  The embedding, final norm and LM head are the target's.  Same
    seeded N(0, 0.02^2) recipe and storage formats as the target's weights."""
    H, D = cfg.hidden, cfg.head_dim
    mc = mtp_config(cfg)
    I = mc.dense_inter
    out = {"enorm": _gain(cfg, H, device, "mtp.enorm"), "hnorm": _gain(cfg, H, device, "mtp.hnorm")}
    out["eh_proj"], out["s_eh_proj"] = _linear(cfg, (H, 2 * H), device, "mtp.eh_proj")
    L = {"attn_norm": _gain(cfg, H, device, "mtp.attn_norm"),
         "ffn_norm": _gain(cfg, H, device, "mtp.ffn_norm")}
    L["w_qkv"], L["s_qkv"] = _linear(cfg, (cfg.qkv_dim, H), device, "mtp.w_qkv")
    L["w_o"], L["s_o"] = _linear(cfg, (H, cfg.n_q * D), device, "mtp.w_o")
    L["w_gate_up"], L["s_gate_up"] = _linear(cfg, (2 * I, H), device, "mtp.w_gate_up")
    L["w_down"], L["s_down"] = _linear(cfg, (H, I), device, "mtp.w_down")
    out["block"] = L
    return out


def mtp_config(cfg: VerifyConfig) -> VerifyConfig:
    """Shape of the FastMTP draft block as a one-layer dense model sharing the
    target's attention shape, vocabulary, K and storage types (an MXFP4 LM
    head stays MXFP4: it is the target's)."""
    import dataclasses
    I = cfg.dense_inter if cfg.ffn == "dense" and cfg.dense_inter else 4 * cfg.hidden
    return dataclasses.replace(cfg, name=cfg.name + "_mtp", n_layers=1, ffn="dense", dense_inter=I,
                               n_experts=0, expert_inter=0, top_k=0, n_shared=0)


def mtp_model_weights(target: dict, mtp: dict) -> dict:
    """The draft block as a weight dict of a one-layer model: the block layer
    with the target's embedding, final norm and LM head (tied)."""
    return {"embed": target["embed"], "layers": [mtp["block"]], "final_norm": target["final_norm"],
            "lm_head": target["lm_head"], "lm_scale": target.get("lm_scale")}
