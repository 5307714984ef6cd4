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


@pytest.mark.parametrize("batch", [16, 40, 64, 5])
def test_mxfp4_many_rows(H, batch):
    """64, 160 and 256 verified rows: the large-row kernel (activation chunks
    in LDS) for the grouped experts (16- and, at 256 rows, 32-row expert
    tiles) and the LM head, with MXFP4 weights; and 20 rows (the few-row
    LM head with two row fragments)."""
    cfg = workloads.scaled(workloads.get_config("moe_b1_mxfp4"), n_layers=2, batch=batch,
                           vocab=4112, ctx=("uniform", 5, 300), norm_gain_std=0.2)
    stats, _ = _run(H, cfg, f"mxfp4_many_rows_b{batch}")
    assert stats["argmax_agree"] >= 0.9 * stats["positions"]


@pytest.mark.parametrize("rows,cols", [(40, 1280), (16, 896), (3, 128)])
def test_pack_mx_scales_layout(H, rows, cols):
    """The tiled scale layout against its definition, element by element."""
    import numpy as np
    import speculative_decoding_verify_step_amd as sv
    g = torch.Generator().manual_seed(rows + cols)
    src = torch.randint(0, 255, (rows, cols // 32), generator=g, dtype=torch.int32).to(torch.uint8)
    got = sv.pack_mx_scales(src.to("cuda")).cpu().numpy()
    steps = cols // 128
    nchunk = (steps + 15) // 16
    nblk = (rows + 15) // 16
    want = np.full((nblk, nchunk, 64, 16), 127, np.uint8)
    s = src.numpy()
    for rb in range(nblk):
        for c in range(nchunk):
            for l in range(64):
                r, gq = 16 * rb + (l & 15), l >> 4
                for j in range(16):
                    st = 16 * c + j
                    if r < rows and st < steps:
                        want[rb, c, l, j] = s[r, 4 * st + gq]
    assert got.shape[0] == want.size
    np.testing.assert_array_equal(got, want.reshape(-1))
