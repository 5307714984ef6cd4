"""Model and workload shapes of the verify-step workloads.

Shapes follow what the pages say about the target decoder:
  * Jina-OCR-v1 paper, abstract and section 3 (Table 1 text): a DeepSeekMoE
    decoder of about 3B parameters with about 570M active per token, behind a
    K=3 FastMTP draft head (section 3.1).
  * jina-ocr-v1 tweet digest: 64 routed + 2 shared experts with top-6
    routing; a 1024x1024 page is 256 vision tokens; a 57.6% draft acceptance
    rate with 2.7 tokens committed per verify.
  * Jina-OCR-v1 release article: 1,085 output tokens per page at
    concurrency 32.
  * OCRia-1 report digest ("three things"): 5k-12k-token synthetic tables;
    block drafts of 31 tokens; concurrency 64.
The per-layer sizes (hidden 1280, 10 heads x 128, expert intermediate 896,
vocab 129,280) make a 12-layer stack of 3.14B parameters with 575M active per
token, matching the paper's totals.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field


@dataclass(frozen=True)
class VerifyConfig:
    name: str
    n_layers: int
    hidden: int
    n_q: int
    n_kv: int
    head_dim: int
    ffn: str                      # "moe" or "dense"
    vocab: int
    batch: int
    k_draft: int
    wdtype: str                   # storage of linear weights: "f32" | "bf16" | "fp8"
    kvdtype: str                  # KV cache storage: "f32" | "bf16"
    embdtype: str                 # embedding table storage: "f32" | "bf16"
    ctx: tuple                    # ("fixed", n) | ("uniform", lo, hi) | ("loguniform", lo, hi)
    draft_p: tuple                # ("const", p) | ("per_seq_uniform", lo, hi) | ("decay", p0, r)
    n_experts: int = 0
    expert_inter: int = 0
    top_k: int = 0
    n_shared: int = 0
    dense_inter: int = 0
    steps: int = 1                # chained verify steps the workload runs
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    renorm_topk: int = 0
    seed: int = 0
    weight_std: float = 0.02
    norm_gain_std: float = 0.0    # 0: gains are exactly 1
    mx: str = ""                  # "mxfp4": experts and LM head in OCP MXFP4 (others per wdtype)
    description: str = field(default="", compare=False)

    @property
    def rows(self) -> int:
        """Verified positions per step, T = B (K + 1)."""
        return self.batch * (self.k_draft + 1)

    @property
    def qkv_dim(self) -> int:
        return (self.n_q + 2 * self.n_kv) * self.head_dim


CONFIGS = {
    "tiny_fp32": VerifyConfig(
        name="tiny_fp32", n_layers=1, hidden=256, n_q=4, n_kv=4, head_dim=64, ffn="moe",
        n_experts=8, expert_inter=128, top_k=2, n_shared=1, vocab=1024, batch=1, k_draft=3,
        wdtype="f32", kvdtype="f32", embdtype="f32", ctx=("fixed", 256), draft_p=("const", 0.6),
        description="1 MoE layer, hidden 256, fp32, batch 1, context 256, K=3"),
    "moe_b1": VerifyConfig(
        name="moe_b1", n_layers=1, hidden=1280, n_q=10, n_kv=10, head_dim=128, ffn="moe",
        n_experts=64, expert_inter=896, top_k=6, n_shared=2, vocab=129280, batch=1, k_draft=3,
        wdtype="bf16", kvdtype="bf16", embdtype="bf16", ctx=("fixed", 1341),
        draft_p=("const", 0.576),
        description="1 MoE layer + LM head, bf16, batch 1, context 1341 (256 vision + 1085 text), K=3"),
    "moe_b32": VerifyConfig(
        name="moe_b32", n_layers=12, hidden=1280, n_q=10, n_kv=10, head_dim=128, ffn="moe",
        n_experts=64, expert_inter=896, top_k=6, n_shared=2, vocab=129280, batch=32, k_draft=3,
        wdtype="bf16", kvdtype="bf16", embdtype="bf16", ctx=("uniform", 300, 2500),
        draft_p=("per_seq_uniform", 0.4, 0.8),
        description="12 MoE layers, bf16, batch 32, contexts U[300,2500], K=3"),
    "dense_fp8_b8": VerifyConfig(
        name="dense_fp8_b8", n_layers=8, hidden=2560, n_q=32, n_kv=8, head_dim=128, ffn="dense",
        dense_inter=9728, vocab=151936, batch=8, k_draft=31, wdtype="fp8", kvdtype="bf16",
        embdtype="bf16", ctx=("uniform", 1500, 6000), draft_p=("decay", 0.85, 0.97),
        description="8 dense GQA layers, fp8 e4m3 weights, batch 8, contexts U[1500,6000], K=31"),
    "moe_b64_long": VerifyConfig(
        name="moe_b64_long", n_layers=12, hidden=1280, n_q=10, n_kv=10, head_dim=128, ffn="moe",
        n_experts=64, expert_inter=896, top_k=6, n_shared=2, vocab=129280, batch=64, k_draft=3,
        wdtype="bf16", kvdtype="bf16", embdtype="bf16", ctx=("loguniform", 1000, 12000),
        draft_p=("const", 0.576), steps=100,
        description="12 MoE layers, bf16, batch 64, contexts log-U[1000,12000], K=3, 100 chained steps"),
    # the batch-1 workload with the weight-streaming matrices (experts, LM
    # head) in OCP MXFP4: gfx950 widens E2M1 with a block scale exactly to
    # bf16; about a quarter of the bf16 bytes
    "moe_b1_mxfp4": VerifyConfig(
        name="moe_b1_mxfp4", n_layers=1, hidden=1280, n_q=10, n_kv=10, head_dim=128, ffn="moe",
        n_experts=64, expert_inter=896, top_k=6, n_shared=2, vocab=129280, batch=1, k_draft=3,
        wdtype="bf16", kvdtype="bf16", embdtype="bf16", ctx=("fixed", 1341),
        draft_p=("const", 0.576), mx="mxfp4",
        description="moe_b1 with MXFP4 experts and LM head (bf16 attention, router, embedding)"),
    "moe_b32_mxfp4": VerifyConfig(
        name="moe_b32_mxfp4", n_layers=12, hidden=1280, n_q=10, n_kv=10, head_dim=128, ffn="moe",
        n_experts=64, expert_inter=896, top_k=6, n_shared=2, vocab=129280, batch=32, k_draft=3,
        wdtype="bf16", kvdtype="bf16", embdtype="bf16", ctx=("uniform", 300, 2500),
        draft_p=("per_seq_uniform", 0.4, 0.8), mx="mxfp4",
        description="moe_b32 with MXFP4 experts and LM head"),
}

# index of each workload in the order the workload list gives them
ORDER = ["tiny_fp32", "moe_b1", "moe_b32", "dense_fp8_b8", "moe_b64_long"]


def get_config(name_or_index) -> VerifyConfig:
    if isinstance(name_or_index, int):
        return CONFIGS[ORDER[name_or_index]]
    return CONFIGS[name_or_index]


def scaled(cfg: VerifyConfig, **overrides) -> VerifyConfig:
    """A copy of `cfg` with some fields replaced (reduced-size parity cases)."""
    if "name" not in overrides:
        overrides["name"] = cfg.name + "_scaled"
    return dataclasses.replace(cfg, **overrides)
