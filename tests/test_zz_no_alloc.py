"""spec_verify_step_noalloc (the verify step for callers that cannot allocate
device memory: its workspace is the library's static device scratch) against
spec_verify_step on the same inputs: accepted lengths, bonus tokens and new
context lengths bit-exact, the written cache slots within the float
tolerance, on two calls in a row (the second with a smaller batch), then a
batch-1 call at the batch-1 workload's full size; a configuration whose
workspace exceeds the scratch is refused on the host; device-side errors
reach the caller's error word."""
import ctypes

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 5e-2}


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_decoding_verify_step_amd as sv
    sv.load_library()
    return sv


def say(*a):
    print(*a, flush=True)


def _noalloc(sv, vctx, kc, vc, com, dr, ci, co, B, acc, nxt, err=None):
    lib = sv.load_library()
    return lib.spec_verify_step_noalloc(
        ctypes.byref(vctx._config), ctypes.byref(vctx._w), kc.data_ptr(), vc.data_ptr(),
        com.data_ptr(), dr.data_ptr(), ci.data_ptr(), co.data_ptr(), int(B), acc.data_ptr(),
        nxt.data_ptr(), None if err is None else err.data_ptr(),
        torch.cuda.current_stream().cuda_stream)


def _greedy_drafts(cfg, vctx, kc0, vc0, com, dr, ci):
    """Drafts that follow the target's greedy tokens (from untimed passes of
    the context step) in even sequences and stay random in odd ones, so that
    both short and full acceptances occur."""
    i32 = dict(dtype=torch.int32, device="cuda")
    B, K = dr.shape
    tgt = torch.empty(B, K + 1, **i32)
    vctx.set_debug(None, None, tgt)
    d = dr.clone()
    kc, vc = kc0.clone(), vc0.clone()
    tmp = [torch.empty(B, **i32) for _ in range(3)]
    for i in range(K):
        vctx.step(kc, vc, com, d, ci, tmp[0], tmp[1], tmp[2])
        d[0::2, i] = tgt[0::2, i]
    vctx.set_debug()
    torch.cuda.synchronize()
    return d


def _compare(sv, cfg, vctx, kc0, vc0, com, dr, ci, B, label):
    """The existing entry point and the no-alloc one from the same caches."""
    i32 = dict(dtype=torch.int32, device="cuda")
    outs = []
    for which in ("context", "noalloc"):
        kc, vc = kc0.clone(), vc0.clone()
        acc, nxt, co = (torch.full((B,), -9, **i32) for _ in range(3))
        err = torch.zeros(1, **i32)
        if which == "context":
            vctx.step(kc, vc, com[:B], dr[:B], ci[:B], co, acc, nxt, batch=B)
        else:
            rc = _noalloc(sv, vctx, kc, vc, com, dr, ci, co, B, acc, nxt, err)
            assert rc == sv.SV_OK, sv.spec_verify_last_error()
        torch.cuda.synchronize()
        if which == "noalloc":
            assert int(err.item()) == 0
        outs.append((acc.cpu(), nxt.cpu(), co.cpu(), kc, vc))
    (a0, n0, c0, k0, v0), (a1, n1, c1, k1, v1) = outs
    say(f"[{label}] B={B} accepted {a0.tolist()[:8]}")
    assert torch.equal(a0, a1) and torch.equal(n0, n1) and torch.equal(c0, c1)
    tol = TOL[cfg.wdtype]
    kn0, vn0 = sv.kv_from_library(k0, v0)
    kn1, vn1 = sv.kv_from_library(k1, v1)
    K1 = cfg.k_draft + 1
    bitwise = True
    for b in range(B):
        c = int(ci[b])
        for x0, x1 in ((kn0, kn1), (vn0, vn1)):
            s0 = x0[b, :, :, c:c + K1].float()
            s1 = x1[b, :, :, c:c + K1].float()
            rng = float(s0.max() - s0.min())
            assert float((s0 - s1).abs().max()) <= tol * rng
            bitwise = bitwise and torch.equal(s0, s1)
    # nothing outside the written slots differs
    for x0, x1 in ((kn0, kn1), (vn0, vn1)):
        y0, y1 = x0.clone(), x1.clone()
        for b in range(B):
            c = int(ci[b])
            y0[b, :, :, c:c + K1] = 0
            y1[b, :, :, c:c + K1] = 0
        assert torch.equal(y0, y1)
    say(f"[{label}] written slots bit-identical: {bitwise}")


def test_noalloc_matches_context_step_twice_then_batch1(sv):
    cfg = workloads.scaled(workloads.get_config("moe_b32"), n_layers=2, vocab=8192, batch=20,
                           ctx=("uniform", 30, 700))
    cap = workloads.capacity_for(cfg)
    w = workloads.make_weights(cfg, "cuda")
    kn, vn = workloads.kv_cache(cfg, "cuda", capacity=cap)
    kc0, vc0 = sv.kv_to_library(kn, vn)
    vctx = sv.VerifyContext(cfg, cfg.batch, cap, w)
    i32 = dict(dtype=torch.int32, device="cuda")
    com = workloads.committed_tokens(cfg).to(**i32)
    ci = workloads.context_lengths(cfg).to(**i32)
    _, rtok = workloads.draft_randomness(cfg)
    dr = _greedy_drafts(cfg, vctx, kc0, vc0, com, rtok[0].to(**i32).contiguous(), ci)
    say(f"[noalloc] {cfg.name}: batch 20 (80 rows, large-row kernels), then batch 3")
    _compare(sv, cfg, vctx, kc0, vc0, com, dr, ci, 20, "noalloc b20")
    _compare(sv, cfg, vctx, kc0, vc0, com, dr, ci, 3, "noalloc b3")
    vctx.close()
    del kc0, vc0, kn, vn, w
    torch.cuda.empty_cache()

    cfg = workloads.get_config("moe_b1")
    cap = workloads.capacity_for(cfg)
    w = workloads.make_weights(cfg, "cuda")
    kn, vn = workloads.kv_cache(cfg, "cuda", capacity=cap)
    kc0, vc0 = sv.kv_to_library(kn, vn)
    vctx = sv.VerifyContext(cfg, 1, cap, w)
    com = workloads.committed_tokens(cfg).to(**i32)
    ci = workloads.context_lengths(cfg).to(**i32)
    _, rtok = workloads.draft_randomness(cfg)
    dr = _greedy_drafts(cfg, vctx, kc0, vc0, com, rtok[0].to(**i32).contiguous(), ci)
    say("[noalloc] moe_b1 full size")
    _compare(sv, cfg, vctx, kc0, vc0, com, dr, ci, 1, "noalloc moe_b1")
    vctx.close()


def test_noalloc_refuses_oversized_and_reports_device_errors(sv):
    # the batch-64 long-context workload needs far more than the scratch: refused
    # on the host, before any launch
    big = workloads.get_config("moe_b64_long")
    conf = sv.make_config(big, big.batch, workloads.capacity_for(big))
    lib = sv.load_library()
    rc = lib.spec_verify_step_noalloc(ctypes.byref(conf), None, None, None, None, None, None, None,
                                      big.batch, None, None, None, None)
    assert rc == sv.SV_ERR_UNSUPPORTED
    assert "scratch" in sv.spec_verify_last_error()
    # a token outside the vocabulary: -1 outputs, the caller's error word set
    cfg = workloads.scaled(workloads.get_config("tiny_fp32"), batch=2)
    cap = workloads.capacity_for(cfg)
    w = workloads.make_weights(cfg, "cuda")
    kn, vn = workloads.kv_cache(cfg, "cuda", capacity=cap)
    kc, vc = sv.kv_to_library(kn, vn)
    vctx = sv.VerifyContext(cfg, 2, cap, w)
    i32 = dict(dtype=torch.int32, device="cuda")
    com = workloads.committed_tokens(cfg).to(**i32)
    com[1] = cfg.vocab + 3
    ci = workloads.context_lengths(cfg).to(**i32)
    dr = workloads.draft_randomness(cfg)[1][0].to(**i32).contiguous()
    acc, nxt, co = (torch.full((2,), -9, **i32) for _ in range(3))
    err = torch.zeros(1, **i32)
    say("[noalloc] bad token in sequence 1")
    assert _noalloc(sv, vctx, kc, vc, com, dr, ci, co, 2, acc, nxt, err) == sv.SV_OK
    torch.cuda.synchronize()
    assert int(err.item()) & sv.SV_DEV_BAD_TOKEN
    assert acc[1].item() == -1 and nxt[1].item() == -1 and co[1].item() == ci[1].item()
    assert acc[0].item() >= 0 and co[0].item() == ci[0].item() + acc[0].item() + 1
    vctx.close()
