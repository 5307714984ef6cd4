"""The C-ABI library builds, loads and exports what include/spec_verify.h
declares; host-side validation works without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_(?:verify|draft)_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def sv():
    import speculative_decoding_verify_step_amd as sv
    from speculative_decoding_verify_step_amd import _build
    if not os.path.exists(sv.LIB_PATH):
        _build.build()
    sv.load_library()
    return sv


def test_every_declared_function_is_exported(sv):
    names = _declared()
    assert len(names) >= 10
    lib = ctypes.CDLL(sv.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(sv.EXPORTS) == names


def test_status_strings_and_version(sv):
    assert sv.spec_verify_abi_version() == 5
    assert sv.spec_verify_status_string(0) == "ok"
    assert "invalid" in sv.spec_verify_status_string(-1)
    assert sv.spec_verify_status_string(12345) == "unknown status"


def test_struct_sizes_match_header(sv):
    # 21 four-byte fields; layer = 16 pointers; weights = 5 pointers + int (padded)
    assert ctypes.sizeof(sv.SpecVerifyConfig) == 24 * 4
    assert ctypes.sizeof(sv.SpecVerifyLayer) == 16 * 8
    assert ctypes.sizeof(sv.SpecVerifyWeights) == 6 * 8


def test_tiled16_sizes(sv):
    assert sv.spec_verify_tiled16_bytes(129280, 1280, sv.SV_BF16) == 129280 * 1280 * 2
    assert sv.spec_verify_tiled16_bytes(8, 256, sv.SV_F32) == 16 * 256 * 4      # padded rows
    assert sv.spec_verify_tiled16_bytes(0, 256, sv.SV_F32) == -1
    lib = sv.load_library()
    assert lib.spec_verify_pack_tiled16(None, None, 16, 64, 1, None) == sv.SV_ERR_INVALID_ARG


def _cfg(sv, **kw):
    import workloads
    c = sv.make_config(workloads.get_config("moe_b1"), 1, 1408)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value", [("head_dim", 96), ("vocab", 1000), ("kv_capacity", 1400),
                                         ("n_kv_heads", 3), ("k_draft", 0), ("kv_dtype", 0),
                                         ("ffn_kind", 7), ("top_k", 9)])
def test_init_rejects_bad_configs_before_touching_the_device(sv, field, value):
    lib = sv.load_library()
    h = ctypes.c_void_p()
    rc = lib.spec_verify_init(ctypes.byref(_cfg(sv, **{field: value})), ctypes.byref(h))
    assert rc == sv.SV_ERR_UNSUPPORTED
    assert h.value is None
    assert sv.spec_verify_last_error()


def test_null_arguments_are_rejected(sv):
    lib = sv.load_library()
    assert lib.spec_verify_init(None, None) == sv.SV_ERR_INVALID_ARG
    assert lib.spec_verify_step(None, None, None, None, None, None, None, None, 1, None, None,
                                None) == sv.SV_ERR_INVALID_ARG
    assert lib.spec_verify_set_debug(None, None, None, None, None) == sv.SV_ERR_INVALID_ARG
    lib.spec_verify_destroy(None)


def test_init_without_gpu_reports_no_device(sv):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    lib = sv.load_library()
    h = ctypes.c_void_p()
    assert lib.spec_verify_init(ctypes.byref(_cfg(sv)), ctypes.byref(h)) == sv.SV_ERR_NO_DEVICE


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_kv_layout_permutation_matches_documented_formulas(sv, dtype, D):
    """kv_to_library places K[pos][d] and V[pos][d] at the element offsets the
    header documents, and kv_from_library inverts it."""
    import torch
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    KL = 8 if dtype == "bf16" else 4
    KT, NB, DS = 4 * KL, KL // 4, D // (4 * KL)
    cap = 128
    # integer tags of the same element size: K holds pos * D + d, V its negative - 1
    itype = torch.int16 if dtype == "bf16" else torch.int32
    idx = torch.arange(cap * D, dtype=torch.int64).reshape(1, 1, 1, cap, D)
    k_lib, v_lib = sv.kv_to_library(idx.to(itype), (-idx - 1).to(itype))
    kf, vf = k_lib.reshape(-1), v_lib.reshape(-1)
    for pos in (0, 1, 5, 8, 13, 31, 32, 77, cap - 1):
        for d in (0, 1, 7, 8, 15, 16, 33, D - 1):
            t, r = pos // KT, pos % KT
            rem = r % KL
            q4, blk = 4 * (r // KL) + rem % 4, rem // 4
            s_, g, e = d // (4 * KL), (d % (4 * KL)) // KL, d % KL
            ko = (((t * NB + blk) * DS + s_) * 64 + q4 + 16 * g) * KL + e
            assert kf[ko].item() == pos * D + d
            g2, e2 = r // KL, r % KL
            vo = ((t * (D // 16) + d // 16) * 64 + d % 16 + 16 * g2) * KL + e2
            assert vf[vo].item() == -(pos * D + d) - 1
    x = torch.randn(2, 3, 2, cap, D).to(tdt)
    y = torch.randn(2, 3, 2, cap, D).to(tdt)
    k2, v2 = sv.kv_from_library(*sv.kv_to_library(x, y))
    assert torch.equal(k2, x) and torch.equal(v2, y)


@pytest.mark.parametrize("B,L,H,order_seed", [(1, 3, 2, 0), (2, 1, 4, 1), (3, 2, 1, None)])
def test_paged_pool_layout(sv, B, L, H, order_seed):
    """kv_paged_from_library: the pool is contiguous and page-major; physical
    page table[b][i] holds logical page i of sequence b, for every (layer,
    head), element for element."""
    import numpy as np
    import torch
    cap, D, page = 256, 64, 64
    npg = cap // page
    k = torch.randn(B, L, H, cap, D)
    v = torch.randn(B, L, H, cap, D)
    order = None if order_seed is None else np.random.default_rng(order_seed).permutation(B * npg)
    kp, vp, table = sv.kv_paged_from_library(k, v, page, order)
    assert kp.is_contiguous() and kp.shape == (B * npg, L, H, page, D)
    flat_k, flat_v = kp.reshape(-1), vp.reshape(-1)
    for b in range(B):
        for i in range(npg):
            pg = int(table[b, i])
            for l in range(L):
                for h in range(H):
                    off = ((pg * L + l) * H + h) * page * D
                    want_k = k[b, l, h, i * page:(i + 1) * page].reshape(-1)
                    want_v = v[b, l, h, i * page:(i + 1) * page].reshape(-1)
                    assert torch.equal(flat_k[off:off + page * D], want_k)
                    assert torch.equal(flat_v[off:off + page * D], want_v)
