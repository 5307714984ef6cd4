"""bench.py host logic without a GPU: the one-GPU refusal, the algorithmic
byte model behind the roofline figures, and the rule that measured HBM
traffic is reported only for the kernel sources it was measured on."""
import json
import os
import subprocess
import sys

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_lm_head_bytes_batch1():
    """129,280 x 1,280 bf16 weights, 4 bf16 activation rows, one 8-byte key
    per 64-column tile and row: the 331,031,680 bytes the roofline uses."""
    cfg = workloads.get_config("moe_b1")
    want = 129280 * 1280 * 2 + 4 * 1280 * 2 + 2020 * 4 * 8
    assert want == 331_031_680
    assert bench.lm_head_bytes(cfg, 4) == want
    # sampled verification also writes the fp32 logits
    assert bench.lm_head_bytes(cfg, 4, logits=True) == want + 4 * 129280 * 4


def test_lm_head_bytes_fp8_and_mxfp4():
    fp8 = workloads.get_config("dense_fp8_b8")
    V, H, T = fp8.vocab, fp8.hidden, 256
    assert bench.lm_head_bytes(fp8, T) == V * H + V * 4 + T * H * 2 + ((V + 63) // 64) * T * 8
    mx = workloads.get_config("moe_b1_mxfp4")
    V, H = mx.vocab, mx.hidden
    # half a byte per code plus one E8M0 scale byte per 32 codes
    assert bench.lm_head_bytes(mx, 4) == V * H // 2 + V * H // 32 + 4 * H * 2 + ((V + 63) // 64) * 4 * 8


def test_step_bytes_batch1_by_hand():
    """One MoE layer at batch 1: attention weights, router, the distinct routed
    experts plus the shared ones, the LM head, the embedding rows, the cached
    context read once and the new K/V written."""
    cfg = workloads.get_config("moe_b1")
    H, D, I = cfg.hidden, cfg.head_dim, cfg.expert_inter
    qkv = (cfg.n_q + 2 * cfg.n_kv) * D
    distinct = 17
    attn = (qkv * H + H * cfg.n_q * D) * 2
    router = cfg.n_experts * H * 2
    experts = (distinct + cfg.n_shared) * 3 * H * I * 2
    lm = cfg.vocab * H * 2
    emb = 4 * H * 2
    kv = (1341 + 4) * 2 * cfg.n_kv * D * 2 + 4 * 2 * cfg.n_kv * D * 2
    want = attn + router + experts + lm + emb + kv
    assert bench.step_bytes(cfg, [1341], [distinct]) == want
    assert want == 481_889_280       # the default benchmark line's bytes_per_step


def test_traffic_only_for_the_measured_sources(monkeypatch):
    m = bench.MEASURED_TRAFFIC["moe_b1"]
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: m["source_sha"])
    t = bench.measured_traffic("moe_b1")
    assert t == m["read_bytes"] + m["write_bytes"]
    # the batch-1 LM head moves its algorithmic bytes to within 0.05 %
    cfg = workloads.get_config("moe_b1")
    assert abs(t / bench.lm_head_bytes(cfg, 4) - 1) < 5e-4
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "0" * 16)
    assert bench.measured_traffic("moe_b1") is None
    assert bench.measured_traffic("moe_b32") is None
    assert bench.measured_traffic("tiny_fp32") is None


def test_attention_and_gate_up_bytes_by_hand():
    b64 = workloads.get_config("moe_b64_long")
    # one layer: K and V rows of every (context + K + 1) position, bf16, per KV head; queries once
    ctx_sum = 64 * (4756 + 4)
    want = ctx_sum * 2 * 10 * 128 * 2 + 256 * 10 * 128 * 2
    assert bench.attention_bytes(b64, ctx_sum) == want
    b32 = workloads.get_config("moe_b32")
    H, I, T = 1280, 896, 128
    # 64 routed experts used + 2 shared: gate and up rows once, rows in, SwiGLU out
    want = (64 + 2) * 2 * I * H * 2 + T * H * 2 + (T * 6 + 2 * T) * I * 2
    assert bench.gate_up_bytes(b32, 64) == want
    for name in bench.DOMINANT:
        assert workloads.get_config(name).name == name


def test_attention_kernel_label_follows_the_library_rule():
    """The roofline names the LDS-ring attention kernel where the library
    uses it: bf16 caches with 17 .. 256 query rows per KV head."""
    assert bench.attention_kernel(workloads.get_config("dense_fp8_b8")) == "attn_lds"   # 32 x 4 rows
    for name in ("moe_b1", "moe_b32", "moe_b64_long", "tiny_fp32"):
        assert bench.attention_kernel(workloads.get_config(name)) == "attn_split"
    wide = workloads.scaled(workloads.get_config("dense_fp8_b8"), k_draft=63)   # 64 x 4 = 256 rows
    assert bench.attention_kernel(wide) == "attn_lds"
    wider = workloads.scaled(workloads.get_config("dense_fp8_b8"), k_draft=64)  # 260 rows
    assert bench.attention_kernel(wider) == "attn_split"
