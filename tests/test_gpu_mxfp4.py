"""MXFP4 expert and LM-head weights (OCP MX E2M1 codes with E8M0 block
scales) on the GPU against the oracle, which decodes the same codes exactly
(oracle/oracle.c); comparison rules as for bf16 weights (gpu_harness)."""
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


def _run(H, cfg, label):
    import test_gpu_parity as P
    return P._verify_case(H, cfg, label=label)


def test_mxfp4_batch1_full_size(H):
    stats, _ = _run(H, workloads.get_config("moe_b1_mxfp4"), "moe_b1_mxfp4")
    assert stats["accept_agree"] == 1


@pytest.mark.parametrize("batch,n_experts,top_k,n_shared", [(12, 64, 6, 2), (3, 16, 4, 1)])
def test_mxfp4_batched_scaled(H, batch, n_experts, top_k, n_shared):
    """More rows per expert (permutation path at 48 rows; implied tiles at 12),
    two layers, norm gains away from 1, a ragged vocabulary."""
    cfg = workloads.scaled(workloads.get_config("moe_b1_mxfp4"), n_layers=2, batch=batch,
                           n_experts=n_experts, top_k=top_k, n_shared=n_shared, vocab=4112,
                           ctx=("uniform", 5, 400), norm_gain_std=0.2)
    stats, _ = _run(H, cfg, f"mxfp4_b{batch}_e{n_experts}")
    assert stats["argmax_agree"] >= 0.9 * stats["positions"]


def test_mxfp4_rejects_large_batches(H):
    import speculative_decoding_verify_step_amd as sv
    cfg = workloads.scaled(workloads.get_config("moe_b1_mxfp4"), batch=16)
    with pytest.raises(sv.SpecVerifyError):
        sv.spec_verify_init(sv.make_config(cfg, 16, 1408))
