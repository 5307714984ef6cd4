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
    return sorted(set(re.findall(r"\b(spec_verify_[a-z0-9_]+)\s*\(", text)))


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
    assert sv.spec_verify_abi_version() == 1
    assert sv.spec_verify_status_string(0) == "ok"
    assert "invalid" in sv.spec_verify_status_string(-1)
    assert sv.spec_verify_status_string(12345) == "unknown status"


def test_struct_sizes_match_header(sv):
    # 21 four-byte fields; layer = 16 pointers; weights = 5 pointers + int (padded)
    assert ctypes.sizeof(sv.SpecVerifyConfig) == 21 * 4
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
